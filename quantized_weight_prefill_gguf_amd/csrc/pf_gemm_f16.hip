// Tiled GEMM, f16 leg: fp16 inputs, fp32 accumulation, f32 output
// (v_mfma_f32_16x16x32_f16), the f16 leg of the page "aprender-serve 0.70.2 -
// src/cuda/executor/gdn_prefill_ops.rs" (module doc, group 1, and
// `qwen35_project_rows_f16`): weights and activations rounded to fp16,
// accumulation and output in fp32. Unlike that page nothing is cached or
// converted in HBM: X is rounded to fp16 while it is staged into LDS, and each
// weight block is decoded to fp16 in registers right before the MFMA that eats it.
//
// Workgroup: 256 threads = 4 waves in a 2 x 2 grid; tile MT token rows x NW weight
// rows; each wave owns (MT/2) x (NW/2) of the fp32 accumulators.
// K loop: one 32-weight block per step (one 16x16x32 MFMA per 16x16 tile).
//  - Weight bytes move in chunks of 8 blocks (256 k): a row's chunk is 144 (Q4_0)
//    or 272 (Q8_0) bytes, 16-byte aligned in HBM when k % 256 == 0, so it is copied
//    raw, GGUF AoS as it is, with 16-byte loads into a double-buffered LDS chunk.
//    Each step copies 1/8 of the next chunk.
//  - X moves one step (32 k) at a time: f32 loads, RNE to fp16, stored in LDS in
//    the k order the weight decode produces (double-buffered).
//  - X loads run one step ahead of the step they feed, weight loads two.
// Lane (c, g) of the B operand decodes 8 weights of its column's block: for Q4_0
// the low and high nibbles of qs bytes 4g..4g+3, for Q8_0 the int8 bytes
// 8g..8g+7; X sits in LDS in the same k order, so an A fragment is one 16-byte read.
//
// Large-n shapes (the gate/up SwiGLU) run one workgroup per output tile; narrow
// ones (n = 4096 at T = 512) split K over workgroups that add their partial sums
// into Y with fp32 atomics (PLAIN zero-fills Y first).
#include "pf_device.h"
#include "pf_internal.h"

namespace pf {

namespace {

constexpr int XS = 40;  // LDS halves per staged X row: 32 + 8 pad (80 bytes)

template <int QT> struct ChunkTraits {
    static constexpr int BB = BlockTraits<QT>::BYTES;
    static constexpr int ROW = 8 * BB;      // bytes of one row's chunk (144 / 272)
    static constexpr int U4 = ROW / 16;     // 16-byte pieces per row chunk (9 / 17)
};

// Where the float4 holding k = 4*c4 .. 4*c4+3 of a block lands (in halves, within
// the row's 32-half segment), so that lane group g finds halves 8g .. 8g+7 ready.
template <int QT> __device__ __forceinline__ int x_half_pos(int c4) {
    if constexpr (QT == Q4_0)
        return 8 * (c4 & 3) + 4 * (c4 >> 2);  // stored as (x0, x2, x1, x3)
    else
        return 4 * c4;                         // natural order
}

}  // namespace

// Global weight row of local tile row lr, or -1 past the weight.
template <int EPI, int NW>
__device__ __forceinline__ int f16_weight_row(int tile_n, int lr, int n) {
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

template <int QT, int EPI, int MT, int NW, bool SPLIT>
__global__ __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_f16_kernel(const uint8_t *__restrict__ W, const float *__restrict__ X,
                     float *__restrict__ Y, int n, int k, int T, int tiles_m, int tiles_n,
                     int splits) {
    using CT = ChunkTraits<QT>;
    constexpr int IT = MT / 32;           // 16-row MFMA tiles per wave
    constexpr int JT = NW / 32;           // 16-column MFMA tiles per wave
    constexpr int XF4 = MT / 32;          // X float4 loads per thread per step
    constexpr int WU = (NW * CT::U4 + 7) / 8;       // 16-byte pieces per step (1/8 chunk)
    constexpr int WPT = (WU + 255) / 256;           // pieces per thread per step
    constexpr int WROW = CT::ROW;
    constexpr int WBUF = NW * WROW + 16;            // +16: decode reads one dword past a row

    __shared__ __attribute__((aligned(16))) _Float16 xs[2][MT * XS];
    __shared__ __attribute__((aligned(16))) uint8_t wsm[2][WBUF];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int c = lane & 15, g = lane >> 4;

    // Workgroup -> tile. Dispatch spreads consecutive workgroup ids over the 8 XCDs;
    // remap so that each XCD gets a contiguous run of tiles in which the M tiles of
    // one weight tile are adjacent (they share the weight chunk in that XCD's L2).
    const int total = tiles_m * tiles_n * splits;
    int logical;
    {
        const int id = blockIdx.x;
        const int per = (total + 7) / 8;
        const int xcd = id & 7, slot = id >> 3;
        const int full = total - 8 * (per - 1);  // XCDs that get `per` tiles
        logical = (xcd < full) ? xcd * per + slot : full * per + (xcd - full) * (per - 1) + slot;
    }
    const int tm = logical % tiles_m;
    const int rest = logical / tiles_m;
    const int tn = rest % tiles_n;
    const int split = rest / tiles_n;
    const int m0 = tm * MT;
    const int nchunks = k >> 8;
    const int c_begin = (int)((long)nchunks * split / splits);
    const int c_end = (int)((long)nchunks * (split + 1) / splits);
    const int nsteps = 8 * (c_end - c_begin);
    const int nb = k >> 5;
    const size_t row_bytes = (size_t)nb * CT::BB;

    // ---- per-thread staging assignments (fixed over the K loop). Every global
    // load is unconditional so the wait counters stay exact: rows past T (X) or
    // past the weight read a valid row instead; such rows only feed outputs that
    // are never stored.
    const float *xsrc[XF4];
    int xdst[XF4];
#pragma unroll
    for (int i = 0; i < XF4; ++i) {
        const int row = (tid >> 3) + 32 * i;
        const int c4 = tid & 7;
        const int t = min(m0 + row, T - 1);
        xsrc[i] = X + (size_t)t * k + 4 * c4;
        xdst[i] = row * XS + x_half_pos<QT>(c4);
    }
    // Weight pieces: slice s of a chunk is pieces [s*WU, (s+1)*WU); piece u is row
    // u / U4, 16-byte piece u % U4. wdst = this thread's index within a slice.
    int wdst[WPT];
#pragma unroll
    for (int i = 0; i < WPT; ++i) wdst[i] = (tid + 256 * i < WU) ? tid + 256 * i : -1;

    // ---- B-operand rows of this wave's column tiles
    int brow[JT];
#pragma unroll
    for (int j = 0; j < JT; ++j) {
        if constexpr (EPI == EPI_SWIGLU) {
            constexpr int HALF = NW / 2, PER = JT / 2 * 16;
            brow[j] = (j < JT / 2) ? wn * PER + j * 16 + c : HALF + wn * PER + (j - JT / 2) * 16 + c;
        } else {
            brow[j] = wn * (JT * 16) + j * 16 + c;
        }
    }

    f4_t acc[IT][JT];
#pragma unroll
    for (int i = 0; i < IT; ++i)
#pragma unroll
        for (int j = 0; j < JT; ++j) acc[i][j] = f4_t{0.f, 0.f, 0.f, 0.f};

    f4_t xr[1][XF4];
    u4_t wr[2][WPT];

    auto x_load = [&](int step, f4_t *dst) __attribute__((always_inline)) {
        const int koff = (c_begin * 8 + step) * 32;
#pragma unroll
        for (int i = 0; i < XF4; ++i) dst[i] = *reinterpret_cast<const f4_t *>(xsrc[i] + koff);
    };
    auto x_store = [&](const f4_t *src, int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < XF4; ++i) {
            const f4_t v = src[i];
            h2_t p0, p1;
            if constexpr (QT == Q4_0) {
                p0 = h2_t{(_Float16)v[0], (_Float16)v[2]};
                p1 = h2_t{(_Float16)v[1], (_Float16)v[3]};
            } else {
                p0 = h2_t{(_Float16)v[0], (_Float16)v[1]};
                p1 = h2_t{(_Float16)v[2], (_Float16)v[3]};
            }
            *reinterpret_cast<u2_t *>(&xs[buf][xdst[i]]) = u2_t{h2_bits(p0), h2_bits(p1)};
        }
    };
    const int last_chunk = c_end - c_begin - 1;
    // Slice `slice` (0..7) of chunk `chunk` (relative to c_begin) into registers.
    // Out-of-range pieces, rows or chunks load a valid address and are not stored.
    auto w_load = [&](int chunk, int slice, u4_t *dst) __attribute__((always_inline)) {
        const int ch = min(chunk, last_chunk);
#pragma unroll
        for (int i = 0; i < WPT; ++i) {
            const int u = min(slice * WU + max(wdst[i], 0), NW * CT::U4 - 1);
            const int lr = u / CT::U4, piece = u % CT::U4;
            int gr = f16_weight_row<EPI, NW>(tn, lr, n);
            gr = gr < 0 ? 0 : gr;
            dst[i] = *reinterpret_cast<const u4_t *>(W + (size_t)gr * row_bytes +
                                                      (size_t)(c_begin + ch) * WROW + 16 * piece);
        }
    };
    auto w_store = [&](int chunk, int slice, const u4_t *src) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < WPT; ++i) {
            const int u = slice * WU + wdst[i];
            if (wdst[i] >= 0 && u < NW * CT::U4 && chunk <= last_chunk) {
                const int lr = u / CT::U4, piece = u % CT::U4;
                *reinterpret_cast<u4_t *>(&wsm[chunk & 1][lr * WROW + 16 * piece]) = src[i];
            }
        }
    };

    // One K step: A fragments from LDS, B fragments decoded from the raw chunk.
    auto compute = [&](int step) __attribute__((always_inline)) {
        const int xb = step & 1;
        const int chunk = step >> 3;
        const int blk = step & 7;
        const uint8_t *wb = wsm[chunk & 1];
        h8_t a[IT];
#pragma unroll
        for (int i = 0; i < IT; ++i)
            a[i] = *reinterpret_cast<const h8_t *>(&xs[xb][(wm * IT * 16 + i * 16 + c) * XS + 8 * g]);
#pragma unroll
        for (int j = 0; j < JT; ++j) {
            const int base = brow[j] * WROW + blk * CT::BB;
            const uint32_t d16 = *reinterpret_cast<const uint16_t *>(wb + base);
            const h2_t d2 = as_h2(d16 | (d16 << 16));
            uint32_t p[4];
            if constexpr (QT == Q4_0) {
                const int addr = base + 2 + 4 * g;  // qs bytes 4g .. 4g+3
                const uint32_t *al = reinterpret_cast<const uint32_t *>(wb + (addr & ~3));
                const uint32_t w = (uint32_t)((((uint64_t)al[1] << 32) | al[0]) >> (8 * (addr & 3)));
                q4_word_to_h8(w, d2, p);
            } else {
                const int addr = base + 2 + 8 * g;  // qs bytes 8g .. 8g+7
                const uint32_t *al = reinterpret_cast<const uint32_t *>(wb + (addr & ~3));
                const int sh = 8 * (addr & 3);
                const uint32_t w0 = (uint32_t)((((uint64_t)al[1] << 32) | al[0]) >> sh);
                const uint32_t w1 = (uint32_t)((((uint64_t)al[2] << 32) | al[1]) >> sh);
                q8_word_to_h4(w0, d2, p);
                q8_word_to_h4(w1, d2, p + 2);
            }
            const h8_t b = __builtin_bit_cast(h8_t, u4_t{p[0], p[1], p[2], p[3]});
#pragma unroll
            for (int i = 0; i < IT; ++i)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[i], b, acc[i][j], 0, 0, 0);
        }
    };

    if (nsteps > 0) {
        // ---- prologue: chunk 0 whole and X for step 0 in LDS; X for step 1 and
        // the weight slices for steps 0, 1 (chunk 1) in registers.
        for (int s = 0; s < 8; ++s) {
            w_load(0, s, wr[0]);
            w_store(0, s, wr[0]);
        }
        x_load(0, xr[0]);
        x_store(xr[0], 0);
        x_load(min(1, nsteps - 1), xr[0]);
        w_load(1, 0, wr[0]);
        w_load(1, 1, wr[1]);
        __syncthreads();

        // Step kb: X(kb+1) sits in xr[0]; the weight slice for step kb (chunk kb/8
        // + 1, slice kb%8) in wr[0], the one for step kb+1 in wr[1]. X is fetched
        // one step ahead, weights two.
        for (int kb = 0; kb < nsteps; ++kb) {
            if (kb + 1 < nsteps) x_store(xr[0], (kb + 1) & 1);
            x_load(min(kb + 2, nsteps - 1), xr[0]);
            w_store((kb >> 3) + 1, kb & 7, wr[0]);
#pragma unroll
            for (int i = 0; i < WPT; ++i) wr[0][i] = wr[1][i];
            w_load(((kb + 2) >> 3) + 1, (kb + 2) & 7, wr[1]);
            compute(kb);
            __syncthreads();
        }
    }

    // ---- epilogue. Lane (c, g) holds D[4g + r][c] of each 16 x 16 tile.
    constexpr int JO = (EPI == EPI_SWIGLU) ? JT / 2 : JT;
#pragma unroll
    for (int i = 0; i < IT; ++i) {
#pragma unroll
        for (int j = 0; j < JO; ++j) {
            int o;
            if constexpr (EPI == EPI_SWIGLU)
                o = tn * (NW / 2) + wn * (JT / 2 * 16) + j * 16 + c;
            else
                o = tn * NW + wn * (JT * 16) + j * 16 + c;
            if (o >= n) continue;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = m0 + wm * IT * 16 + i * 16 + 4 * g + r;
                if (t >= T) continue;
                float *y = Y + (size_t)t * n + o;
                if constexpr (EPI == EPI_SWIGLU) {
                    *y = silu_f32(acc[i][j][r]) * acc[i][j + JT / 2][r];
                } else if constexpr (SPLIT) {
                    atomicAdd(y, acc[i][j][r]);
                } else if constexpr (EPI == EPI_PLAIN) {
                    *y = acc[i][j][r];
                } else {
                    *y = *y + acc[i][j][r];
                }
            }
        }
    }
}

__global__ void zero_fill_kernel(float *__restrict__ Y, int count) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < count) Y[i] = 0.f;
}

namespace {

struct TileChoice {
    int cfg;     // 0: 256x192, 1: 256x128, 2: 128x128, 3: 64x64
    int splits;
};

constexpr int CFG_MT[4] = {256, 256, 128, 64};
constexpr int CFG_NW[4] = {192, 128, 128, 64};
// Relative MFMA efficiency of each tile shape (bigger wave tiles feed the matrix
// cores with fewer LDS bytes and decode instructions per flop).
constexpr float CFG_EFF[4] = {1.0f, 0.92f, 0.75f, 0.35f};

TileChoice choose_tiles(const GemmArgs &a) {
    const bool swiglu = a.epilogue == EPI_SWIGLU;
    const long n_w = swiglu ? 2L * a.n : a.n;
    const int nchunks = a.k / 256;
    const int cus = 256;
    TileChoice best{3, 1};
    float best_t = 1e30f;
    for (int cfg = 0; cfg < 4; ++cfg) {
        const int MT = CFG_MT[cfg], NW = CFG_NW[cfg];
        const long out_per_tile = swiglu ? NW / 2 : NW;
        const long tm = (a.T + MT - 1) / MT;
        const long tn = (a.n + out_per_tile - 1) / out_per_tile;
        for (int s = 1; s <= 8; ++s) {
            if (s > 1 && (swiglu || s > nchunks)) break;
            const long wgs = tm * tn * s;
            const long rounds = (wgs + cus - 1) / cus;
            // time ~ rounds x work per workgroup / efficiency, plus a split-K cost
            const float work = (float)MT * NW * ((float)a.k / s);
            float t = rounds * work / CFG_EFF[cfg];
            if (s > 1) t *= 1.0f + 0.02f * s;
            (void)n_w;
            if (t < best_t) {
                best_t = t;
                best = TileChoice{cfg, s};
            }
        }
    }
    return best;
}

template <int QT, int EPI, int MT, int NW, bool SPLIT>
hipError_t launch_cfg(const GemmArgs &a, int splits, hipStream_t s) {
    constexpr int OUT = (EPI == EPI_SWIGLU) ? NW / 2 : NW;
    const int tm = (a.T + MT - 1) / MT;
    const int tn = (a.n + OUT - 1) / OUT;
    const int total = tm * tn * splits;
    hipLaunchKernelGGL((gemm_f16_kernel<QT, EPI, MT, NW, SPLIT>), dim3(total), dim3(256), 0, s,
                       a.W, a.X, a.Y, a.n, a.k, a.T, tm, tn, splits);
    return hipGetLastError();
}

template <int QT, int EPI, bool SPLIT>
hipError_t launch_split(const GemmArgs &a, TileChoice tc, hipStream_t s) {
    switch (tc.cfg) {
    case 0: return launch_cfg<QT, EPI, 256, 192, SPLIT>(a, tc.splits, s);
    case 1: return launch_cfg<QT, EPI, 256, 128, SPLIT>(a, tc.splits, s);
    case 2: return launch_cfg<QT, EPI, 128, 128, SPLIT>(a, tc.splits, s);
    default: return launch_cfg<QT, EPI, 64, 64, SPLIT>(a, tc.splits, s);
    }
}

template <int QT, int EPI>
hipError_t launch_epi(const GemmArgs &a, hipStream_t s) {
    const TileChoice tc = choose_tiles(a);
    if constexpr (EPI == EPI_SWIGLU) {
        return launch_split<QT, EPI, false>(a, TileChoice{tc.cfg, 1}, s);
    } else {
        if (tc.splits == 1) return launch_split<QT, EPI, false>(a, tc, s);
        if constexpr (EPI == EPI_PLAIN) {
            const int count = a.T * a.n;
            hipLaunchKernelGGL(zero_fill_kernel, dim3((count + 255) / 256), dim3(256), 0, s, a.Y, count);
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
        return launch_split<QT, EPI, true>(a, tc, s);
    }
}

template <int QT>
hipError_t launch_q(const GemmArgs &a, hipStream_t s) {
    switch (a.epilogue) {
    case EPI_PLAIN: return launch_epi<QT, EPI_PLAIN>(a, s);
    case EPI_RESIDUAL: return launch_epi<QT, EPI_RESIDUAL>(a, s);
    default: return launch_epi<QT, EPI_SWIGLU>(a, s);
    }
}

}  // namespace

hipError_t launch_gemm_f16(const GemmArgs &a, hipStream_t s) {
    return a.qtype == Q4_0 ? launch_q<Q4_0>(a, s) : launch_q<Q8_0>(a, s);
}

}  // namespace pf
