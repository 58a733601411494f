// Tiled GEMM, f32 leg: Y = epilogue(X . W_hat^T) with exact f32 weights, f32
// activations and fp32 matrix-core accumulation (v_mfma_f32_16x16x4_f32, no
// reduced-precision inputs), as the page "aprender-serve 0.70.2 -
// src/cuda/executor/gdn_prefill_ops.rs" (module doc, group 1) asks of the f32 leg:
// fp32 in and out with no TF32.
//
// Workgroup: 256 threads = 4 waves in a 2 x 2 grid; tile MT token rows x NW weight
// rows; K advances one 32-weight block per step. Each step stages the X tile (f32)
// and the raw weight blocks in LDS (double-buffered, one barrier per step); each
// wave decodes its weight columns from LDS into registers and feeds the MFMA.
// The weight stays in GGUF AoS form in HBM and is never expanded there.
#include "pf_device.h"
#include "pf_internal.h"

namespace pf {

namespace {

constexpr int F32_MT = 64;  // token rows per workgroup
constexpr int F32_NW = 64;  // weight rows per workgroup
constexpr int F32_WM = 2;   // 16-row MFMA tiles per wave along M
constexpr int F32_WN = 2;   // 16-column MFMA tiles per wave along N
constexpr int F32_XS = 36;  // LDS floats per staged X row (32 + 4 pad)

// LDS bytes per staged block: 2 bytes of padding so that the qs bytes start
// 4-byte aligned, the 2-byte scale, then the qs bytes.
template <int QT> constexpr int slot_bytes() { return QT == Q4_0 ? 20 : 36; }

}  // namespace

// Global weight row of local tile row lr; -1 if it lies past the weight.
template <int EPI, int NW>
__device__ __forceinline__ int tile_weight_row(int tile_n, int lr, int n) {
    if constexpr (EPI == EPI_SWIGLU) {
        constexpr int HALF = NW / 2;
        const int o = tile_n * HALF + (lr % HALF);
        if (o >= n) return -1;
        return lr < HALF ? o : n + o;
    } else {
        const int r = tile_n * NW + lr;
        return r < n ? r : -1;
    }
}

template <int QT, int EPI>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const uint8_t *__restrict__ W,
                                                       const float *__restrict__ X,
                                                       float *__restrict__ Y, int n, int ldy,
                                                       int k, int T) {
    constexpr int MT = F32_MT, NW = F32_NW, WM = F32_WM, WN = F32_WN, XS = F32_XS;
    constexpr int BB = BlockTraits<QT>::BYTES;
    constexpr int HW = BlockTraits<QT>::HALFWORDS;
    constexpr int SLOT = slot_bytes<QT>();
    constexpr int X_F4 = MT * 8 / 256;              // float4 X loads per thread per step
    constexpr int W_HW = (NW * HW + 255) / 256;     // u16 weight loads per thread per step

    __shared__ float xs[2][MT * XS];
    __shared__ __attribute__((aligned(16))) uint8_t ws[2][NW * SLOT];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int c = lane & 15, g = lane >> 4;
    const int tile_n = blockIdx.x;
    const int m0 = blockIdx.y * MT;
    const int nb = k >> 5;

    // Per-thread staging assignments (fixed over the K loop).
    int x_row[X_F4], x_c4[X_F4];
#pragma unroll
    for (int i = 0; i < X_F4; ++i) {
        const int idx = tid + 256 * i;
        x_row[i] = idx >> 3;
        x_c4[i] = idx & 7;
    }
    int w_lr[W_HW], w_u[W_HW];
    const uint8_t *w_src[W_HW];
#pragma unroll
    for (int i = 0; i < W_HW; ++i) {
        const int idx = tid + 256 * i;
        w_lr[i] = idx / HW;
        w_u[i] = idx % HW;
        const int gr = (idx < NW * HW) ? tile_weight_row<EPI, NW>(tile_n, w_lr[i], n) : -1;
        w_src[i] = gr >= 0 ? W + (size_t)gr * nb * BB + 2 * w_u[i] : nullptr;
    }

    f4_t xr[X_F4];
    uint16_t wr[W_HW];
    auto load_step = [&](int kb) {
#pragma unroll
        for (int i = 0; i < X_F4; ++i) {
            const int t = m0 + x_row[i];
            xr[i] = t < T ? *reinterpret_cast<const f4_t *>(X + (size_t)t * k + kb * 32 + 4 * x_c4[i])
                          : f4_t{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int i = 0; i < W_HW; ++i)
            wr[i] = w_src[i] ? *reinterpret_cast<const uint16_t *>(w_src[i] + (size_t)kb * BB) : 0;
    };
    auto store_step = [&](int buf) {
#pragma unroll
        for (int i = 0; i < X_F4; ++i)
            *reinterpret_cast<f4_t *>(&xs[buf][x_row[i] * XS + 4 * x_c4[i]]) = xr[i];
#pragma unroll
        for (int i = 0; i < W_HW; ++i)
            if (tid + 256 * i < NW * HW)
                *reinterpret_cast<uint16_t *>(&ws[buf][w_lr[i] * SLOT + 2 + 2 * w_u[i]]) = wr[i];
    };

    // Local weight rows of this wave's MFMA column tiles.
    int b_lr[WN];
#pragma unroll
    for (int j = 0; j < WN; ++j) {
        if constexpr (EPI == EPI_SWIGLU) {
            constexpr int HALF = NW / 2, PER = WN / 2 * 16;
            b_lr[j] = (j < WN / 2) ? wn * PER + j * 16 + c : HALF + wn * PER + (j - WN / 2) * 16 + c;
        } else {
            b_lr[j] = wn * (WN * 16) + j * 16 + c;
        }
    }

    f4_t acc[WM][WN];
#pragma unroll
    for (int i = 0; i < WM; ++i)
#pragma unroll
        for (int j = 0; j < WN; ++j) acc[i][j] = f4_t{0.f, 0.f, 0.f, 0.f};

    load_step(0);
    store_step(0);
    __syncthreads();

    for (int kb = 0; kb < nb; ++kb) {
        const int buf = kb & 1;
        if (kb + 1 < nb) load_step(kb + 1);

        // A operand: lane (row c, group g) takes the 8 k-slots of its group.
        float a[WM][8];
#pragma unroll
        for (int i = 0; i < WM; ++i) {
            const float *row = &xs[buf][(wm * WM * 16 + i * 16 + c) * XS];
            f4_t lo, hi;
            if constexpr (QT == Q4_0) {
                lo = *reinterpret_cast<const f4_t *>(row + 4 * g);
                hi = *reinterpret_cast<const f4_t *>(row + 16 + 4 * g);
            } else {
                lo = *reinterpret_cast<const f4_t *>(row + 8 * g);
                hi = *reinterpret_cast<const f4_t *>(row + 8 * g + 4);
            }
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                a[i][s] = lo[s];
                a[i][4 + s] = hi[s];
            }
        }
        // B operand: the same 8 k-slots of weight column c, decoded exactly.
        float b[WN][8];
#pragma unroll
        for (int j = 0; j < WN; ++j) {
            const uint8_t *slot = &ws[buf][b_lr[j] * SLOT];
            const float d = fp16_bits_to_f32(*reinterpret_cast<const uint16_t *>(slot + 2));
            if constexpr (QT == Q4_0) {
                const uint32_t w = *reinterpret_cast<const uint32_t *>(slot + 4 + 4 * g);
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    b[j][s] = q4_nibble_f32(w, 8 * s, d);          // k = 4g + s
                    b[j][4 + s] = q4_nibble_f32(w, 8 * s + 4, d);  // k = 16 + 4g + s
                }
            } else {
                const uint32_t w0 = *reinterpret_cast<const uint32_t *>(slot + 4 + 8 * g);
                const uint32_t w1 = *reinterpret_cast<const uint32_t *>(slot + 8 + 8 * g);
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    b[j][s] = q8_byte_f32(w0, s, d);      // k = 8g + s
                    b[j][4 + s] = q8_byte_f32(w1, s, d);  // k = 8g + 4 + s
                }
            }
        }
#pragma unroll
        for (int s = 0; s < 8; ++s)
#pragma unroll
            for (int i = 0; i < WM; ++i)
#pragma unroll
                for (int j = 0; j < WN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i][s], b[j][s], acc[i][j], 0, 0, 0);

        if (kb + 1 < nb) store_step(buf ^ 1);
        __syncthreads();
    }

    // Epilogue. Lane (c, g) holds D[4g + r][c] of each 16 x 16 tile.
    constexpr int JO = (EPI == EPI_SWIGLU) ? WN / 2 : WN;
#pragma unroll
    for (int i = 0; i < WM; ++i) {
#pragma unroll
        for (int j = 0; j < JO; ++j) {
            int o;
            if constexpr (EPI == EPI_SWIGLU)
                o = tile_n * (NW / 2) + wn * (WN / 2 * 16) + j * 16 + c;
            else
                o = tile_n * NW + wn * (WN * 16) + j * 16 + c;
            if (o >= n) continue;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = m0 + wm * WM * 16 + i * 16 + 4 * g + r;
                if (t >= T) continue;
                float *y = Y + (size_t)t * ldy + o;
                if constexpr (EPI == EPI_PLAIN) {
                    *y = acc[i][j][r];
                } else if constexpr (EPI == EPI_RESIDUAL) {
                    *y = *y + acc[i][j][r];
                } else {
                    *y = silu_f32(acc[i][j][r]) * acc[i][j + WN / 2][r];
                }
            }
        }
    }
}

template <int QT, int EPI>
static hipError_t launch_f32_typed(const GemmArgs &a, hipStream_t s) {
    constexpr int OUT_PER_TILE = (EPI == EPI_SWIGLU) ? F32_NW / 2 : F32_NW;
    const dim3 grid((a.n + OUT_PER_TILE - 1) / OUT_PER_TILE, (a.T + F32_MT - 1) / F32_MT);
    hipLaunchKernelGGL((gemm_f32_kernel<QT, EPI>), grid, dim3(256), 0, s, a.W, a.X, a.Y, a.n, a.ldy, a.k,
                       a.T);
    return hipGetLastError();
}

template <int QT>
static hipError_t launch_f32_q(const GemmArgs &a, hipStream_t s) {
    switch (a.epilogue) {
    case EPI_PLAIN: return launch_f32_typed<QT, EPI_PLAIN>(a, s);
    case EPI_RESIDUAL: return launch_f32_typed<QT, EPI_RESIDUAL>(a, s);
    default: return launch_f32_typed<QT, EPI_SWIGLU>(a, s);
    }
}

hipError_t launch_gemm_f32(const GemmArgs &a, hipStream_t s) {
    return a.qtype == Q4_0 ? launch_f32_q<Q4_0>(a, s) : launch_f32_q<Q8_0>(a, s);
}

}  // namespace pf
