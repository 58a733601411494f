// Internal interface between the C ABI (pf_api.cpp) and the kernel launchers.
// Host-only types; the launchers live next to their kernels in the .hip files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pf {

// One validated GEMM call. Element counts fit in 31 bits (checked by the API).
struct GemmArgs {
    int qtype;      // PF_Q4_0 / PF_Q8_0
    int epilogue;   // PF_PLAIN / PF_RESIDUAL / PF_GATE_UP_SWIGLU
    const uint8_t *W;
    const float *X;
    float *Y;
    int n;          // output columns
    int ldy;        // floats between consecutive rows of Y (>= n)
    int k;          // reduction length, multiple of 256
    int T;          // token rows, >= 1
    // RMSNorm prologue for the f16 workspace path (both null: none): X is read as
    // X[t][j] * norm_inv[t] * norm_w[j].
    const float *norm_w = nullptr;
    const float *norm_inv = nullptr;
};

// Tiled matrix-core GEMM, f32 leg (fp32 MFMA).
hipError_t launch_gemm_f32(const GemmArgs &a, hipStream_t s);
// Tiled matrix-core GEMM, f16 leg (fp16 MFMA, fp32 accumulation).
hipError_t launch_gemm_f16(const GemmArgs &a, hipStream_t s);
// The same with a caller workspace: X is converted to fp16 once into it (in the
// order the A fragments take), then the GEMM streams fp16 X. The workspace holds
// T * k halves.
hipError_t launch_gemm_f16_ws(const GemmArgs &a, void *workspace, hipStream_t s);
// The two halves of launch_gemm_f16_ws: X to binary16 into the workspace, then the
// GEMM on that copy.
hipError_t launch_prepare_x_f16(const GemmArgs &a, void *workspace, hipStream_t s);
hipError_t launch_gemm_f16_prepared(const GemmArgs &a, void *workspace, hipStream_t s);
// Workspace bytes launch_gemm_f16_ws takes for qtype: X as binary16 (T rounded up to a
// multiple of 32), and with a K split, behind it (at the next 256-byte boundary) one
// [T][n] f32 block of partial sums per split (or G's blocks for SwiGLU up to 64 rows).
int64_t f16_ws_bytes(int qtype, int T, int n, int k, int epilogue);
// The further types the f16 workspace path's GEMMs take (Q4_K, Q5_K and IQ4_XS at every
// T: the 4-wave kernel below 256 rows, the cooperative-decode kernel from 256; F16, and
// Q6_K with k % 512 == 0, from 512); the others keep their own GEMM.
bool f16_takes_xq(int qtype, int T, int k);
// The further types the f16 GEMM without a workspace takes (launch_gemm_f16: Q4_K, Q5_K,
// IQ4_XS, and Q6_K with k % 512 == 0); the others keep their own GEMM there.
bool f16_direct_takes_xq(int qtype, int k);
// Floats between the [T][n] partial-sum blocks of a K split, and Y = [R +] the `splits`
// blocks at ps added in split order (PLAIN or RESIDUAL; a.Y, a.ldy, a.T, a.n).
long part_stride(int T, int n);
hipError_t launch_split_sum(const GemmArgs &a, const float *ps, int splits, hipStream_t s);
// Y [T][n] (a.Y, a.ldy) = silu(g) * u from the `splits` blocks G_s [T][2n] at G
// (part_stride(T, 2n) floats apart; gate products in columns 0..n-1, up in n..2n-1),
// each sum in split order.
hipError_t launch_swiglu_apply(const float *G, const GemmArgs &a, int splits, hipStream_t s);
// RMSNorm prologue: inv[t] = 1 / sqrt(mean_j X[t][j]^2 + eps) (T workgroups), and
// Xn[t][j] = X[t][j] * inv[t] * w[j] for the kernels that read f32 X.
hipError_t launch_rms_inv(const float *X, int T, int k, float eps, float *inv, hipStream_t s);
hipError_t launch_rms_apply(const float *X, const float *inv, const float *w, float *Xn, int T, int k,
                            hipStream_t s);
// token[0] = the largest index among the maxima of logits[0 .. n) (one workgroup).
hipError_t launch_argmax(const float *logits, int n, int32_t *token, hipStream_t s);
// Small-T GEMV (T <= 8), f32 arithmetic on the vector ALU.
hipError_t launch_gemv(const GemmArgs &a, hipStream_t s);
// Small-T GEMV (T <= 8) on the fp32 matrix cores (exact f32 operands).
hipError_t launch_gemv_mfma(const GemmArgs &a, hipStream_t s);
// Size of the static device scratch pf_gemm_noalloc runs in (PF_NOALLOC_SCRATCH_BYTES),
// and its address on the device of stream s (taken once per device, then cached).
constexpr int64_t kNoallocScratchBytes = int64_t(64) << 20;
hipError_t noalloc_scratch(hipStream_t s, void **ptr);
// The further weight types (ids as the C ABI's PF_F16 .. PF_IQ4_XS), pf_xq.hip: the
// GEMV (T <= 8, f32), the tiled GEMM on either leg (leg16: binary16 operands), and
// the block decode to f32 or binary16 bits.
enum { XQ_F16 = 2, XQ_Q4_K = 3, XQ_Q5_K = 4, XQ_Q6_K = 5, XQ_IQ4_XS = 6 };
hipError_t launch_xq_gemv(const GemmArgs &a, hipStream_t s);
// ws: room for xq_ws_bytes() of the call, or null (then nothing splits).
hipError_t launch_xq_gemm(const GemmArgs &a, bool leg16, void *ws, hipStream_t s);
// Workspace bytes of the further types' own GEMM on the f16 leg: the partial sums of a
// K split where PLAIN / RESIDUAL tiles leave CUs idle, else 0.
int64_t xq_ws_bytes(int T, int n, int k, int epilogue, bool leg16);
hipError_t launch_xq_dequant(int qtype, const uint8_t *W, int rows, int k, void *out, bool f16_out,
                             hipStream_t s);
// Block decode to f32 / binary16.
hipError_t launch_dequant_f32(int qtype, const uint8_t *W, int rows, int k, float *out,
                              hipStream_t s);
hipError_t launch_dequant_f16(int qtype, const uint8_t *W, int rows, int k, uint16_t *out,
                              hipStream_t s);

}  // namespace pf
