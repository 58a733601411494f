// Small-T twin of the GEMM (1 <= T <= 8). The weight stream is the cost: every
// weight block is read from HBM once, decoded in registers and applied to all T
// activation rows. This is the kernel-level form of the single-token
// `gemv_q4_0_pf` / `gemv_q8_0_pf` on the page "oxibonsai-kernels 0.1.4 -
// src/gpu_backend/cuda_q_std_prefill.rs", widened to up to 8 rows (the same page's
// batch tests step tokens 8 at a time).
//
// Work split. A wave owns a group of R weight rows (R outputs, or R/2 outputs with
// their gate and up rows for the SwiGLU epilogue) over the whole reduction;
// persistent workgroups of four waves walk super-groups of four groups. Lanes own
// block pairs: lane l takes pair l of each 64-pair step (a pair is 36 bytes for
// Q4_0, 68 for Q8_0). A wave reads its rows' step in coalesced 16-byte chunks into
// its own LDS region and each lane then takes its pair's dwords from there; x is
// staged in LDS once per workgroup (lane-transposed, so that a wave's reads are
// consecutive) and, for one step of few tokens, kept in registers.
//
// Arithmetic (f32 throughout, both legs). With u the unsigned code of a weight
// (the nibble for Q4_0, the int8 byte + 128 for Q8_0) and c its offset (8 or 128),
// w = d (u - c) exactly, and per block
//     sum_j w_j x_j = d (sum_j u_j x_j - c sum_j x_j),
// which costs one integer-to-float conversion and one FMA per weight and token;
// sum_j x_j is shared by the R rows. Only the rounding order differs from
// decoding w first; the bound is the f32 leg's.
//
// The R * T partial sums are combined across the 64 lanes by a butterfly that
// halves the number of values a lane carries at every step.
#include "pf_device.h"
#include "pf_internal.h"

namespace pf {

namespace {

template <int QT> struct PairTraits;
template <> struct PairTraits<Q4_0> {
    static constexpr int DW = 9;         // 36 bytes
    static constexpr int WORDS = 4;      // qs words per block, 8 weights each
    static constexpr float OFF = 8.0f;
};
template <> struct PairTraits<Q8_0> {
    static constexpr int DW = 17;        // 68 bytes
    static constexpr int WORDS = 8;      // qs words per block, 4 weights each
    static constexpr float OFF = 128.0f;
};

typedef uint32_t u4a_t __attribute__((ext_vector_type(4), aligned(4)));
typedef float f4a_t __attribute__((ext_vector_type(4), aligned(16)));

// One pair step of a row is up to 64 consecutive pairs: up to 2304 (Q4_0) or 4352
// (Q8_0) contiguous bytes, a multiple of 16 since rows hold a multiple of 4 pairs.
// A wave reads it in 16-byte chunks, consecutive lanes taking consecutive chunks
// (NCH loads per lane, the last partly duplicated), and parks it in its own LDS
// region, from which each lane then takes the dwords of its pair.
template <int QT> struct StepTraits {
    static constexpr int PB = PairTraits<QT>::DW * 4;      // bytes per pair
    static constexpr int CHUNKS = 64 * PB / 16;            // 16-byte chunks per full step
    static constexpr int NCH = (CHUNKS + 63) / 64;         // chunk loads per lane
    static constexpr int ROW_LDS = NCH * 64 * 16;          // LDS bytes per row (padded)
};

// Block h (0 or 1) of a pair: its scale and qs word m. Block 0 starts at byte 0 of
// the pair (qs at bytes 2 .., straddling dwords), block 1 at byte DW*2 (its qs
// dword-aligned).
template <int QT>
__device__ __forceinline__ float pair_scale(const uint32_t (&dw)[PairTraits<QT>::DW], int h) {
    constexpr int MID = PairTraits<QT>::DW / 2;  // dword holding block 1's scale (high half)
    return fp16_bits_to_f32(h == 0 ? (dw[0] & 0xFFFFu) : (dw[MID] >> 16));
}
template <int QT>
__device__ __forceinline__ uint32_t pair_word(const uint32_t (&dw)[PairTraits<QT>::DW], int h, int m) {
    constexpr int MID = PairTraits<QT>::DW / 2;
    if (h == 0) return __builtin_amdgcn_alignbyte(dw[m + 1], dw[m], 2);
    return dw[MID + 1 + m];
}

__device__ __forceinline__ float ubyte_f32(uint32_t w, int b) {
    return (float)((w >> (8 * b)) & 0xFFu);
}

// Sums v[0 .. N) over the 64 lanes. Afterwards lane l holds the total of value
// index l >> (6 - log2 N) in v[0] (N a power of two, at most 64).
template <int N>
__device__ __forceinline__ void wave_reduce_transpose(float (&v)[N], int lane) {
    static_assert(N >= 1 && N <= 64 && (N & (N - 1)) == 0, "N: power of two <= 64");
    int dist = 32;
    int cnt = N;
#pragma unroll
    for (int step = 0; step < 6; ++step, dist >>= 1) {
        if (cnt > 1) {
            const bool upper = (lane & dist) != 0;
            const int half = cnt / 2;
#pragma unroll
            for (int i = 0; i < N / 2; ++i) {
                if (i < half) {
                    const float send = upper ? v[i] : v[i + half];
                    const float keep = upper ? v[i + half] : v[i];
                    v[i] = keep + __shfl_xor(send, dist, 64);
                }
            }
            cnt = half;
        } else {
            v[0] += __shfl_xor(v[0], dist, 64);
        }
    }
}

constexpr int pow2_ceil(int x) { return x <= 1 ? 1 : 2 * pow2_ceil((x + 1) / 2); }
constexpr int ilog2(int x) { return x <= 1 ? 0 : 1 + ilog2(x / 2); }

// x of one pair step (64 pairs = 4096 k) for TT tokens, in LDS as float4 f[t][i][l]
// = x[t][4096 * step + 64 l + 4 i .. + 3]: lane l's 16 float4 (i = 0 .. 15) lie 1 KB
// apart, so a wave reading one i for all lanes touches consecutive 16 bytes. Steps
// held at once follow each other (16 KB per token and step).
__device__ __forceinline__ int x_lds_index(int t, int i, int l) { return (t * 16 + i) * 64 + l; }

// Adds the pair's contribution to acc[t * R + r] for the R rows whose pair dwords
// are in dw; x comes from the step's LDS copy.
// x of a lane's pair held in registers: f[t][i] as in the LDS copy, and the
// two blocks' sums xs[t][h].
template <int TT>
struct PairXRegs {
    f4_t f[TT][16];
    float xs[TT][2];
};

// XS (x from LDS, fixed for the run): the two blocks' sums of x come precomputed in
// xsum[t][h] instead of being added up again for every row.
template <int QT, int TT, int R, bool XR, bool XS>
__device__ __forceinline__ void pair_accumulate(const uint32_t (&dw)[R][PairTraits<QT>::DW],
                                                const f4_t *xl, const PairXRegs<XR ? TT : 1> &xg,
                                                const float (&xsum)[TT][2], int lane, bool valid,
                                                float (&acc)[pow2_ceil(R * TT)]) {
    using PT = PairTraits<QT>;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        float s[R][TT], xs[TT];
#pragma unroll
        for (int t = 0; t < TT; ++t) {
            xs[t] = 0.f;
#pragma unroll
            for (int r = 0; r < R; ++r) s[r][t] = 0.f;
        }
#pragma unroll
        for (int m = 0; m < PT::WORDS; ++m) {
            // Q4_0 word m covers k = 4m .. 4m+3 of the block (low nibbles) and
            // 16+4m .. 16+4m+3 (high nibbles); Q8_0 word m covers 4m .. 4m+3.
            f4_t xa[TT], xb[TT];
#pragma unroll
            for (int t = 0; t < TT; ++t) {
                if constexpr (XR) {
                    xa[t] = xg.f[t][8 * h + m];
                    if constexpr (QT == Q4_0) xb[t] = xg.f[t][8 * h + 4 + m];
                } else {
                    // x summed one element at a time in the order of the FMA chain
                    // below, so that a block whose codes all equal the offset (a
                    // zero weight) gives exactly s == OFF * x_sum, i.e. 0.
                    xa[t] = xl[x_lds_index(t, 8 * h + m, lane)];
                    if constexpr (!XS) {
#pragma unroll
                        for (int b = 0; b < 4; ++b) xs[t] = xs[t] + xa[t][b];
                    }
                    if constexpr (QT == Q4_0) {
                        xb[t] = xl[x_lds_index(t, 8 * h + 4 + m, lane)];
                        if constexpr (!XS) {
#pragma unroll
                            for (int b = 0; b < 4; ++b) xs[t] = xs[t] + xb[t][b];
                        }
                    }
                }
            }
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const uint32_t w = pair_word<QT>(dw[r], h, m);
                float ua[4], ub[4];
                if constexpr (QT == Q4_0) {
                    uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
                    // Opaque to the optimizer, so that each byte converts with a
                    // single v_cvt_f32_ubyteN instead of a bit-field extract first.
                    asm("" : "+v"(lo), "+v"(hi));
#pragma unroll
                    for (int b = 0; b < 4; ++b) {
                        ua[b] = ubyte_f32(lo, b);
                        ub[b] = ubyte_f32(hi, b);
                    }
                } else {
                    const uint32_t u = w ^ 0x80808080u;
#pragma unroll
                    for (int b = 0; b < 4; ++b) ua[b] = ubyte_f32(u, b);
                }
#pragma unroll
                for (int t = 0; t < TT; ++t) {
                    float a = s[r][t];
#pragma unroll
                    for (int b = 0; b < 4; ++b) a = fmaf(ua[b], xa[t][b], a);
                    if constexpr (QT == Q4_0) {
#pragma unroll
                        for (int b = 0; b < 4; ++b) a = fmaf(ub[b], xb[t][b], a);
                    }
                    s[r][t] = a;
                }
            }
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float d = pair_scale<QT>(dw[r], h);
#pragma unroll
            for (int t = 0; t < TT; ++t) {
                const float x_sum = XR ? xg.xs[t][h] : (XS ? xsum[t][h] : xs[t]);
                const float c = d * fmaf(-PT::OFF, x_sum, s[r][t]);
                acc[t * R + r] += valid ? c : 0.f;
            }
        }
    }
}

// LDS of the kernel: x of NXS pair steps, then the weight staging of WV waves.
template <int QT, int TT, int R, int NXS, int WV>
constexpr int gemv_lds_bytes() { return NXS * TT * 16384 + WV * R * StepTraits<QT>::ROW_LDS; }
constexpr int LDS_MAX = 160 * 1024;

// Grid: persistent workgroups of WV waves (4, or 16 where x of a long row would
// otherwise leave few waves per CU). A workgroup takes super-groups sg =
// blockIdx.x, + gridDim.x, ...; wave w of it owns row group WV sg + w (R weight
// rows, OUTW outputs).
// NS >= 1: a row has NS pair steps (k <= 4096 NS) and the x of all of them is
// staged in LDS once, at the start; the waves then run independently.
// NS == 0: x of the whole row does not fit. The waves walk the same
// (super-group, pair step) items in lockstep and each step's x is restaged, for
// all of them at once, per item.
template <int QT, int EPI, int TT, int R, int NS, int WV>
__global__ __launch_bounds__(64 * WV) void gemv_kernel(const uint8_t *__restrict__ W,
                                                   const float *__restrict__ X,
                                                   float *__restrict__ Y, int n, int ldy,
                                                   int k, int ngroups) {
    using PT = PairTraits<QT>;
    using ST = StepTraits<QT>;
    constexpr int OUTW = (EPI == EPI_SWIGLU) ? R / 2 : R;  // outputs per group
    constexpr int NV = pow2_ceil(R * TT);
    constexpr int LG = ilog2(NV);
    constexpr bool MULTI = NS == 0;          // x restaged per item
    constexpr int NXS = MULTI ? 1 : NS;      // steps of x in LDS
    constexpr bool XPRE = MULTI && TT <= 2;  // next step's x prefetched in registers
    constexpr bool XR = NS == 1 && TT <= 2;  // a lane's x fixed for the run: in registers
    static_assert(NV <= 64, "too many partial sums per lane");
    constexpr int NT = 64 * WV;              // threads
    constexpr int XC = 1024 / NT;            // x float4 per thread, token and step
    static_assert(1024 % NT == 0, "x staging");
    static_assert(gemv_lds_bytes<QT, TT, R, NXS, WV>() <= LDS_MAX, "LDS");

    __shared__ __attribute__((aligned(16))) uint8_t smem[gemv_lds_bytes<QT, TT, R, NXS, WV>()];
    f4_t *xl = reinterpret_cast<f4_t *>(smem);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // wave index, known to the compiler as uniform across the wave
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    uint8_t *my_lds = smem + NXS * TT * 16384 + wid * (R * ST::ROW_LDS);

    const int nsg = (ngroups + WV - 1) / WV;
    if ((int)blockIdx.x >= nsg) return;  // whole workgroup leaves together
    const int npairs = k >> 6;
    const int ipg = (npairs + 63) >> 6;  // pair steps per row
    const int total = ((nsg - 1 - (int)blockIdx.x) / (int)gridDim.x + 1) * ipg;
    const size_t row_bytes = (size_t)npairs * ST::PB;

    auto row_of = [&](int sg, int r) __attribute__((always_inline)) {
        const int o = (WV * sg + wid) * OUTW;
        if constexpr (EPI == EPI_SWIGLU)
            return (r < R / 2) ? min(o + r, n - 1) : n + min(o + r - R / 2, n - 1);
        else
            return min(o + r, n - 1);
    };

    // x of pair step `step`: thread tid holds float4 j = tid + NT c of each token's
    // 1024 (pair j >> 4, float4 j & 15); float4s past the row's end are clamped.
    auto load_x = [&](int step, f4_t (&xr)[TT][XC]) __attribute__((always_inline)) {
        const int np = min(64, npairs - 64 * step);
#pragma unroll
        for (int t = 0; t < TT; ++t)
#pragma unroll
            for (int c = 0; c < XC; ++c) {
                const int j = min(tid + NT * c, 16 * np - 1);
                xr[t][c] = *reinterpret_cast<const f4_t *>(X + (size_t)t * k + 4096 * step + 4 * j);
            }
    };
    auto store_x = [&](const f4_t (&xr)[TT][XC], int slot) __attribute__((always_inline)) {
#pragma unroll
        for (int t = 0; t < TT; ++t)
#pragma unroll
            for (int c = 0; c < XC; ++c) {
                const int j = tid + NT * c;
                xl[slot * TT * 1024 + x_lds_index(t, j & 15, j >> 4)] = xr[t][c];
            }
    };

    // Item `it` = pair step it % ipg of super-group blockIdx.x + (it / ipg) *
    // gridDim.x, tracked by counters: one stream for loads, one for compute.
    int lsg = blockIdx.x, lpi = 0, lcount = 0;  // next item to load
    auto load_next = [&](u4_t (&ch)[R][ST::NCH], auto &xr) __attribute__((always_inline)) {
        const int np = min(64, npairs - 64 * lpi);  // pairs in this step
        const int nchunk = np * ST::PB / 16;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const uint8_t *seg = W + (size_t)row_of(lsg, r) * row_bytes + (size_t)lpi * 64 * ST::PB;
#pragma unroll
            for (int c = 0; c < ST::NCH; ++c) {
                const int j = min(lane + 64 * c, nchunk - 1);
                ch[r][c] = *reinterpret_cast<const u4_t *>(seg + 16 * j);
            }
        }
        if constexpr (XPRE) load_x(lpi, xr);
        (void)xr;
        if (lcount + 1 < total) {  // the last item is loaded again, harmlessly
            ++lcount;
            if (++lpi == ipg) {
                lpi = 0;
                lsg += gridDim.x;
            }
        }
    };
    // Chunks -> this wave's LDS region -> the dwords of each lane's pair. Lanes
    // read what other lanes wrote, so wave_lds_sync separates the writes from the
    // reads, and the previous item's reads from these writes: its fences keep the
    // compiler from moving the accesses across, and its s_waitcnt lgkmcnt(0) makes
    // the wave's earlier LDS operations complete before a later one issues.
    auto unpack = [&](const u4_t (&ch)[R][ST::NCH], uint32_t (&dw)[R][PT::DW]) __attribute__((always_inline)) {
        wave_lds_sync();
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int c = 0; c < ST::NCH; ++c)
                *reinterpret_cast<u4_t *>(my_lds + r * ST::ROW_LDS + 16 * (lane + 64 * c)) = ch[r][c];
        wave_lds_sync();
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const uint32_t *src = reinterpret_cast<const uint32_t *>(my_lds + r * ST::ROW_LDS) + PT::DW * lane;
#pragma unroll
            for (int i = 0; i < PT::DW; ++i) dw[r][i] = src[i];
        }
    };

    float acc[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) acc[i] = 0.f;

    PairXRegs<XR ? TT : 1> xg;
    // XS: x of a single pair step stays in LDS for the run; this lane's block sums,
    // once. (With several steps held, selecting the step's sums per item measured
    // slower than adding them up again: Q8_0 4096 x 12288 at T = 2, 22 -> 34 us.)
    constexpr bool XS = !MULTI && !XR && NS == 1;
    float xsp[XS ? NXS : 1][TT][2] = {};
    int csg = blockIdx.x, cpi = 0;  // item being computed
    // x of the item's step into LDS (all four waves take part).
    auto stage_x = [&](const auto &xr) __attribute__((always_inline)) {
        __syncthreads();  // every wave is done with the previous step's x
        if constexpr (XPRE) {
            store_x(xr, 0);
        } else {
            (void)xr;
            f4_t xd[TT][XC];
            load_x(cpi, xd);
            store_x(xd, 0);
        }
        __syncthreads();
    };
    auto compute = [&](const uint32_t (&dw)[R][PT::DW]) __attribute__((always_inline)) {
        const int p = lane + 64 * cpi;
        float cur[TT][2];
#pragma unroll
        for (int t = 0; t < TT; ++t)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                cur[t][h] = xsp[0][t][h];
#pragma unroll
                for (int st = 1; st < (XS ? NXS : 1); ++st)
                    if (cpi == st) cur[t][h] = xsp[st][t][h];
            }
        pair_accumulate<QT, TT, R, XR, XS>(dw, xl + (MULTI ? 0 : cpi * TT * 1024), xg, cur, lane,
                                           p < npairs, acc);
        if (++cpi == ipg) {  // group complete: reduce over the lanes and store
            cpi = 0;
            float v[NV];
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                v[i] = acc[i];
                acc[i] = 0.f;
            }
            wave_reduce_transpose<NV>(v, lane);
            // Lane l now holds the sum for value index idx = t * R + r.
            const int idx = lane >> (6 - LG);
            const bool owner = (lane & ((1 << (6 - LG)) - 1)) == 0;
            float y = v[0];
            if constexpr (EPI == EPI_SWIGLU) {
                // the up sum of slot r sits R/2 value indices higher
                const float u = __shfl_xor(y, (R / 2) << (6 - LG), 64);
                y = silu_f32(y) * u;
            }
            const int t = idx / R, r = idx % R;
            const int o = (WV * csg + wid) * OUTW + r;
            if (owner && idx < R * TT && r < OUTW && o < n) {
                float *dst = Y + (size_t)t * ldy + o;
                if constexpr (EPI == EPI_RESIDUAL)
                    *dst = *dst + y;
                else
                    *dst = y;
            }
            csg += gridDim.x;
        }
    };

    u4_t cha[R][ST::NCH], chb[R][ST::NCH];
    f4_t xra[XPRE ? TT : 1][XC], xrb[XPRE ? TT : 1][XC];
    uint32_t dw[R][PT::DW];
    load_next(cha, xra);  // the first weights are on their way while x is staged
    if constexpr (!MULTI) {
        // x of every pair step, staged once for the whole run (steps past the
        // row's end are never read).
#pragma unroll
        for (int st = 0; st < NS; ++st) {
            if (st < ipg) {
                f4_t xd[TT][XC];
                load_x(st, xd);
                store_x(xd, st);
            }
        }
        __syncthreads();
        if constexpr (XS) {
            // the order of pair_accumulate's FMA chain (see there)
            using PT = PairTraits<QT>;
#pragma unroll
            for (int st = 0; st < NXS; ++st)
#pragma unroll
                for (int t = 0; t < TT; ++t)
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const f4_t *xs_l = xl + st * TT * 1024;
                        float a = 0.f;
#pragma unroll
                        for (int m = 0; m < PT::WORDS; ++m) {
                            const f4_t qa = xs_l[x_lds_index(t, 8 * h + m, lane)];
#pragma unroll
                            for (int b = 0; b < 4; ++b) a = a + qa[b];
                            if constexpr (QT == Q4_0) {
                                const f4_t qb = xs_l[x_lds_index(t, 8 * h + 4 + m, lane)];
#pragma unroll
                                for (int b = 0; b < 4; ++b) a = a + qb[b];
                            }
                        }
                        xsp[st][t][h] = a;
                    }
        }
        if constexpr (XR) {
#pragma unroll
            for (int t = 0; t < TT; ++t) {
#pragma unroll
                for (int i = 0; i < 16; ++i) xg.f[t][i] = xl[x_lds_index(t, i, lane)];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    // the order of pair_accumulate's FMA chain (see there)
                    using PT = PairTraits<QT>;
                    float a = 0.f;
#pragma unroll
                    for (int m = 0; m < PT::WORDS; ++m) {
                        const f4_t qa = xg.f[t][8 * h + m];
#pragma unroll
                        for (int b = 0; b < 4; ++b) a = a + qa[b];
                        if constexpr (QT == Q4_0) {
                            const f4_t qb = xg.f[t][8 * h + 4 + m];
#pragma unroll
                            for (int b = 0; b < 4; ++b) a = a + qb[b];
                        }
                    }
                    xg.xs[t][h] = a;
                }
            }
        }
    }
    for (int it = 0; it < total; it += 2) {
        load_next(chb, xrb);  // weights (and x) of the next item in flight
        if constexpr (MULTI) stage_x(xra);
        unpack(cha, dw);
        compute(dw);
        load_next(cha, xra);
        if (it + 1 < total) {  // uniform across the workgroup
            if constexpr (MULTI) stage_x(xrb);
            unpack(chb, dw);
            compute(dw);
        }
    }
}

// Workgroups of kernel `kern` (`threads` threads) that fit on one CU at once.
template <typename K>
int resident_blocks_per_cu(K kern, int threads) {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kern, threads, 0) != hipSuccess || nb < 1) nb = 1;
    return nb;
}

template <int QT, int EPI, int TT, int R, int NS, int WV>
hipError_t launch_m(const GemmArgs &a, int ngroups, hipStream_t s) {
    auto kern = gemv_kernel<QT, EPI, TT, R, NS, WV>;
    static const int per_cu = resident_blocks_per_cu(kern, 64 * WV);
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
        cus = 256;
    // Persistent workgroups: one resident round. With four waves each workgroup
    // streams two or more super-groups (x is staged once per workgroup; four per
    // workgroup left the 4096-row weights one workgroup per CU: Q8_0 4096 x 12288 at
    // T = 1 16.2 -> 14.2 us with two, Q4_0 4096 x 12288 13.8 -> 11.4). With sixteen,
    // one or more.
    constexpr int SG_PER_WG = WV == 4 ? 2 : 1;
    const int blocks = min((ngroups + SG_PER_WG * WV - 1) / (SG_PER_WG * WV), per_cu * cus);
    hipLaunchKernelGGL(kern, dim3(blocks), dim3(64 * WV), 0, s, a.W, a.X, a.Y, a.n, a.ldy, a.k, ngroups);
    return hipGetLastError();
}

template <int QT, int EPI, int TT, int R>
hipError_t launch_r(const GemmArgs &a, hipStream_t s) {
    constexpr int OUTW = (EPI == EPI_SWIGLU) ? R / 2 : R;
    const int ngroups = (a.n + OUTW - 1) / OUTW;
    // Stage x of the whole row once when it fits beside the weight staging. Rows of
    // two or three steps stage 32 or 48 KB of x per token: sixteen waves share it
    // where that fits, so that more waves per CU keep weight loads in flight.
    const int steps = (a.k + 4095) / 4096;
    constexpr bool F1 = gemv_lds_bytes<QT, TT, R, 1, 4>() <= LDS_MAX;
    constexpr bool F2 = gemv_lds_bytes<QT, TT, R, 2, 4>() <= LDS_MAX;
    constexpr bool F3 = gemv_lds_bytes<QT, TT, R, 3, 4>() <= LDS_MAX;
    constexpr bool F2W = gemv_lds_bytes<QT, TT, R, 2, 16>() <= LDS_MAX;
    constexpr bool F3W = gemv_lds_bytes<QT, TT, R, 3, 16>() <= LDS_MAX;
    if constexpr (F1)
        if (steps == 1) return launch_m<QT, EPI, TT, R, 1, 4>(a, ngroups, s);
    if constexpr (F2W)
        if (steps == 2) return launch_m<QT, EPI, TT, R, 2, 16>(a, ngroups, s);
    if constexpr (F2)
        if (steps == 2) return launch_m<QT, EPI, TT, R, 2, 4>(a, ngroups, s);
    if constexpr (F3W)
        if (steps == 3) return launch_m<QT, EPI, TT, R, 3, 16>(a, ngroups, s);
    if constexpr (F3)
        if (steps == 3) return launch_m<QT, EPI, TT, R, 3, 4>(a, ngroups, s);
    return launch_m<QT, EPI, TT, R, 0, 4>(a, ngroups, s);
}

// Rows per group: one for PLAIN / RESIDUAL with up to four tokens (x is read
// from registers or LDS, so sharing it buys little, while the smaller weight
// staging and register use let more waves keep loads in flight: measured 11.2 ->
// 9.9 us at T = 1 on Q4_0 12288 x 4096), else two (the SwiGLU gate/up pair, or
// the FMAs of many tokens).
template <int QT, int EPI, int TT>
hipError_t launch_t(const GemmArgs &a, hipStream_t s) {
    if constexpr (EPI != EPI_SWIGLU && TT <= 4) return launch_r<QT, EPI, TT, 1>(a, s);
    return launch_r<QT, EPI, TT, 2>(a, s);
}

// T rows [t0, t0 + tt) as their own problem.
inline GemmArgs token_slice(const GemmArgs &a, int t0, int tt) {
    GemmArgs b = a;
    b.X = a.X + (size_t)t0 * a.k;
    b.Y = a.Y + (size_t)t0 * a.ldy;
    b.T = tt;
    return b;
}

template <int QT, int EPI>
hipError_t launch_tt(const GemmArgs &a, hipStream_t s) {
    switch (a.T) {
    case 1: return launch_t<QT, EPI, 1>(a, s);
    case 2: return launch_t<QT, EPI, 2>(a, s);
    case 3: return launch_t<QT, EPI, 3>(a, s);
    default: return launch_t<QT, EPI, 4>(a, s);
    }
}

// Tokens per launch: at most four (one weight row per group), and at most 96 KB of
// x, so that the chunk's x stays staged in LDS for the whole run beside the weight
// staging. Larger chunks restage x per item or run at lower occupancy; measured on
// Q4_0 12288 x 4096: T = 8 in one launch 55.9 us, as 4 + 4 tokens 43.3 us; Q8_0
// 4096 x 12288 (48 KB of x per token): T = 4 in one launch 56.4 us, as 2 + 2 44 us,
// T = 3 47.3 us against 2 + 1 39.7 us. Rows are independent, so each chunk is its
// own problem; the weights stream once per chunk.
inline int gemv_tokens_per_launch(int k) {
    const int by_x = (96 * 1024) / (k * 4);
    return by_x < 1 ? 1 : (by_x > 4 ? 4 : by_x);
}

template <int QT, int EPI>
hipError_t launch_epi(const GemmArgs &a, hipStream_t s) {
    const int per = gemv_tokens_per_launch(a.k);
    for (int t0 = 0; t0 < a.T; t0 += per) {
        const hipError_t e = launch_tt<QT, EPI>(token_slice(a, t0, min(per, a.T - t0)), s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
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

hipError_t launch_gemv(const GemmArgs &a, hipStream_t s) {
    // 1 <= T <= GEMV_MAX_T is checked by the API.
    return a.qtype == Q4_0 ? launch_q<Q4_0>(a, s) : launch_q<Q8_0>(a, s);
}

}  // namespace pf
