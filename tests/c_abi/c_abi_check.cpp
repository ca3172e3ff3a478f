// Stand-alone check of the C ABI: only include/qf8.h, libqf8.so and the HIP runtime, no Python
// and no torch. Quantizes a seeded BF16 tensor per tensor and MX dual on hipMalloc'd memory,
// de-scales the MX result, and compares every byte (and the fp32 scale/amax bits) with the CPU
// oracle's C functions, linked in from oracle/qf8_oracle.c. Prints "ok" and exits 0 on success.
// Test infrastructure: built by the package build step, run by tests/test_gpu_c_abi.py.
#include <hip/hip_runtime.h>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "../../include/qf8.h"

extern "C" {
void qf8o_quantize_per_tensor(const void *x, int dtype, int64_t rows, int64_t cols, int fmt, uint8_t *q,
                              float *amax_out, float *scale_out, int32_t *nonfinite);
void qf8o_quantize_mx(const void *x, int dtype, int64_t rows, int64_t cols, int fmt, int rnd, uint8_t *q_row,
                      uint8_t *s_row, uint8_t *q_colT, uint8_t *s_colT, int32_t *nonfinite);
void qf8o_dequant_mx(const uint8_t *q, const uint8_t *sb, int64_t rows, int64_t cols, int fmt, float *out);
}

#define HIP_OK(x) do { hipError_t e_ = (x); if (e_ != hipSuccess) { std::printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); return 1; } } while (0)
#define QF8_OK_(x) do { qf8_status s_ = (x); if (s_ != QF8_OK) { std::printf("%s at line %d\n", qf8_status_string(s_), __LINE__); return 1; } } while (0)

static int same(const void *a, const void *b, size_t n, const char *what) {
    if (std::memcmp(a, b, n) == 0) return 0;
    const uint8_t *x = (const uint8_t *)a, *y = (const uint8_t *)b;
    size_t i = 0;
    while (x[i] == y[i]) ++i;
    std::printf("%s differs at byte %zu: %02x vs %02x\n", what, i, x[i], y[i]);
    return 1;
}

int main() {
    const int64_t R = 512, C = 1024, N = R * C;
    // seeded BF16 input: a 32-bit LCG, exponents in [100, 131], random signs and mantissas
    std::vector<uint16_t> h(N);
    uint32_t st = 2024u;
    for (auto &v : h) {
        st = st * 1664525u + 1013904223u;
        v = (uint16_t)(((st >> 8) & 0x8000u) | ((100u + (st >> 27)) << 7) | ((st >> 10) & 0x7Fu));
    }
    void *x, *ws;
    uint8_t *q, *qr, *sr, *qc, *sc;
    float *amax, *scale, *dq;
    const size_t wsb = qf8_workspace_bytes(R, C, QF8_IN_BF16);
    HIP_OK(hipMalloc(&x, N * 2));
    HIP_OK(hipMalloc(&q, N));
    HIP_OK(hipMalloc(&qr, N));
    HIP_OK(hipMalloc(&qc, N));
    HIP_OK(hipMalloc(&sr, N / 32));
    HIP_OK(hipMalloc(&sc, N / 32));
    HIP_OK(hipMalloc(&amax, 4));
    HIP_OK(hipMalloc(&scale, 4));
    HIP_OK(hipMalloc(&dq, N * 4));
    HIP_OK(hipMalloc(&ws, wsb));
    HIP_OK(hipMemcpy(x, h.data(), N * 2, hipMemcpyHostToDevice));
    QF8_OK_(qf8_workspace_init(ws, wsb, nullptr));

    QF8_OK_(quantize_per_tensor(x, QF8_IN_BF16, R, C, QF8_E4M3, q, amax, scale, nullptr, ws, wsb, nullptr));
    QF8_OK_(quantize_mx_dual(x, QF8_IN_BF16, R, C, QF8_E5M2, QF8_MX_ROUND_DOWN, qr, sr, qc, sc, nullptr, nullptr));
    QF8_OK_(dequantize_mx(qr, sr, R, C, QF8_E5M2, dq, QF8_OUT_FP32, nullptr, QF8_IN_BF16, nullptr, nullptr, 0, nullptr));
    HIP_OK(hipDeviceSynchronize());

    std::vector<uint8_t> gq(N), gqr(N), gqc(N), gsr(N / 32), gsc(N / 32), wq(N), wqr(N), wqc(N), wsr(N / 32), wsc(N / 32);
    std::vector<float> gdq(N), wdq(N);
    float ga, gs, wa, wsc_;
    int32_t nf = 0;
    HIP_OK(hipMemcpy(gq.data(), q, N, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(gqr.data(), qr, N, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(gqc.data(), qc, N, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(gsr.data(), sr, N / 32, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(gsc.data(), sc, N / 32, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(gdq.data(), dq, N * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(&ga, amax, 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(&gs, scale, 4, hipMemcpyDeviceToHost));

    qf8o_quantize_per_tensor(h.data(), 0, R, C, 0, wq.data(), &wa, &wsc_, &nf);
    qf8o_quantize_mx(h.data(), 0, R, C, 1, 0, wqr.data(), wsr.data(), wqc.data(), wsc.data(), &nf);
    qf8o_dequant_mx(wqr.data(), wsr.data(), R, C, 1, wdq.data());

    int bad = 0;
    bad |= same(&ga, &wa, 4, "per-tensor amax");
    bad |= same(&gs, &wsc_, 4, "per-tensor scale");
    bad |= same(gq.data(), wq.data(), N, "per-tensor codes");
    bad |= same(gqr.data(), wqr.data(), N, "MX q_row");
    bad |= same(gsr.data(), wsr.data(), N / 32, "MX s_row");
    bad |= same(gqc.data(), wqc.data(), N, "MX q_colT");
    bad |= same(gsc.data(), wsc.data(), N / 32, "MX s_colT");
    bad |= same(gdq.data(), wdq.data(), N * 4, "MX de-scaled fp32");
    // the workspace is back to zero after the single-pass or two-kernel per-tensor call
    std::vector<uint32_t> wsh(wsb / 4);
    HIP_OK(hipMemcpy(wsh.data(), ws, 4 * 32, hipMemcpyDeviceToHost));
    for (int i = 0; i < 32; ++i)
        if (wsh[i] != 0u) { std::printf("workspace header word %d not zero\n", i); bad = 1; }
    for (void *p : {x, (void *)q, (void *)qr, (void *)qc, (void *)sr, (void *)sc, (void *)amax, (void *)scale,
                    (void *)dq, ws})
        HIP_OK(hipFree(p));
    if (bad) return 1;
    std::printf("ok\n");
    return 0;
}
