// Tiled GEMM, f16 leg: fp16 inputs, fp32 accumulation, f32 output
// (v_mfma_f32_16x16x32_f16), as the page "aprender-serve 0.70.2 -
// src/cuda/executor/gdn_prefill_ops.rs" (module doc, group 1, and
// `qwen35_project_rows_f16`) defines the f16 leg: weights and activations rounded
// to fp16, accumulation and output in fp32. Unlike that page, nothing is cached
// or converted in HBM: X is rounded to fp16 while it is staged into LDS, and each
// weight block is decoded to fp16 in registers right before the MFMA.
//
// One 16x16x32 MFMA consumes exactly one 32-weight block per column, so K
// advances one block per step. Lane (c, g) of the B operand decodes 8 weights of
// block (column c): for Q4_0 the low and high nibbles of qs bytes 4g..4g+3, for
// Q8_0 the int8 bytes 8g..8g+7. X is staged in LDS in the same k order, so each
// A fragment is one 16-byte LDS read.
#include "pf_device.h"
#include "pf_internal.h"

namespace pf {

namespace {

constexpr int H_MT = 64;
constexpr int H_NW = 64;
constexpr int H_WM = 2;
constexpr int H_WN = 2;
constexpr int H_XS = 40;  // LDS halves per staged X row (32 + 8 pad): 80 bytes

template <int QT> constexpr int h_slot_bytes() { return QT == Q4_0 ? 20 : 36; }

// Position (in halves, within a 32-half row segment) where the float4 holding
// k = 4*c4 .. 4*c4+3 is stored, and the order of its 4 values, so that lane group
// g finds its 8 values contiguous at halves 8g .. 8g+7.
template <int QT> __device__ __forceinline__ int x_half_pos(int c4) {
    if constexpr (QT == Q4_0)
        return 8 * (c4 & 3) + 4 * (c4 >> 2);  // stored as (x0, x2, x1, x3)
    else
        return 4 * c4;                         // natural order
}

}  // namespace

template <int EPI, int NW>
__device__ __forceinline__ int h_tile_weight_row(int tile_n, int lr, int n) {
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
__global__ __launch_bounds__(256) void gemm_f16_kernel(const uint8_t *__restrict__ W,
                                                       const float *__restrict__ X,
                                                       float *__restrict__ Y, int n, int k,
                                                       int T) {
    constexpr int MT = H_MT, NW = H_NW, WM = H_WM, WN = H_WN, XS = H_XS;
    constexpr int BB = BlockTraits<QT>::BYTES;
    constexpr int HW = BlockTraits<QT>::HALFWORDS;
    constexpr int SLOT = h_slot_bytes<QT>();
    constexpr int X_F4 = MT * 8 / 256;
    constexpr int W_HW = (NW * HW + 255) / 256;

    __shared__ __attribute__((aligned(16))) _Float16 xs[2][MT * XS];
    __shared__ __attribute__((aligned(16))) uint8_t ws[2][NW * SLOT];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int c = lane & 15, g = lane >> 4;
    const int tile_n = blockIdx.x;
    const int m0 = blockIdx.y * MT;
    const int nb = k >> 5;

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
        const int gr = (idx < NW * HW) ? h_tile_weight_row<EPI, NW>(tile_n, w_lr[i], n) : -1;
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
        for (int i = 0; i < X_F4; ++i) {
            const f4_t v = xr[i];
            h2_t p0, p1;
            if constexpr (QT == Q4_0) {
                p0 = h2_t{(_Float16)v[0], (_Float16)v[2]};
                p1 = h2_t{(_Float16)v[1], (_Float16)v[3]};
            } else {
                p0 = h2_t{(_Float16)v[0], (_Float16)v[1]};
                p1 = h2_t{(_Float16)v[2], (_Float16)v[3]};
            }
            uint2 packed = make_uint2(h2_bits(p0), h2_bits(p1));
            *reinterpret_cast<uint2 *>(&xs[buf][x_row[i] * XS + x_half_pos<QT>(x_c4[i])]) = packed;
        }
#pragma unroll
        for (int i = 0; i < W_HW; ++i)
            if (tid + 256 * i < NW * HW)
                *reinterpret_cast<uint16_t *>(&ws[buf][w_lr[i] * SLOT + 2 + 2 * w_u[i]]) = wr[i];
    };

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

        h8_t a[WM];
#pragma unroll
        for (int i = 0; i < WM; ++i)
            a[i] = *reinterpret_cast<const h8_t *>(&xs[buf][(wm * WM * 16 + i * 16 + c) * XS + 8 * g]);

        h8_t b[WN];
#pragma unroll
        for (int j = 0; j < WN; ++j) {
            const uint8_t *slot = &ws[buf][b_lr[j] * SLOT];
            const uint32_t d16 = *reinterpret_cast<const uint16_t *>(slot + 2);
            const h2_t d2 = as_h2(d16 | (d16 << 16));
            uint32_t p[4];
            if constexpr (QT == Q4_0) {
                q4_word_to_h8(*reinterpret_cast<const uint32_t *>(slot + 4 + 4 * g), d2, p);
            } else {
                q8_word_to_h4(*reinterpret_cast<const uint32_t *>(slot + 4 + 8 * g), d2, p);
                q8_word_to_h4(*reinterpret_cast<const uint32_t *>(slot + 8 + 8 * g), d2, p + 2);
            }
            b[j] = __builtin_bit_cast(h8_t, make_uint4(p[0], p[1], p[2], p[3]));
        }
#pragma unroll
        for (int i = 0; i < WM; ++i)
#pragma unroll
            for (int j = 0; j < WN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[i], b[j], acc[i][j], 0, 0, 0);

        if (kb + 1 < nb) store_step(buf ^ 1);
        __syncthreads();
    }

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
                float *y = Y + (size_t)t * n + o;
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
static hipError_t launch_f16_typed(const GemmArgs &a, hipStream_t s) {
    constexpr int OUT_PER_TILE = (EPI == EPI_SWIGLU) ? H_NW / 2 : H_NW;
    const dim3 grid((a.n + OUT_PER_TILE - 1) / OUT_PER_TILE, (a.T + H_MT - 1) / H_MT);
    hipLaunchKernelGGL((gemm_f16_kernel<QT, EPI>), grid, dim3(256), 0, s, a.W, a.X, a.Y, a.n, a.k,
                       a.T);
    return hipGetLastError();
}

template <int QT>
static hipError_t launch_f16_q(const GemmArgs &a, hipStream_t s) {
    switch (a.epilogue) {
    case EPI_PLAIN: return launch_f16_typed<QT, EPI_PLAIN>(a, s);
    case EPI_RESIDUAL: return launch_f16_typed<QT, EPI_RESIDUAL>(a, s);
    default: return launch_f16_typed<QT, EPI_SWIGLU>(a, s);
    }
}

hipError_t launch_gemm_f16(const GemmArgs &a, hipStream_t s) {
    return a.qtype == Q4_0 ? launch_f16_q<Q4_0>(a, s) : launch_f16_q<Q8_0>(a, s);
}

}  // namespace pf
