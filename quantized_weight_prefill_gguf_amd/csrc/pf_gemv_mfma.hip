// Small-T twin of the GEMM on the fp32 matrix cores, for Q4_0 and Q8_0 weights on
// the f32 leg (the C ABI runs it from 3 to 8 token rows): the kernel-level form of
// the single-token `gemv_q4_0_pf` / `gemv_q8_0_pf` on the page "oxibonsai-kernels
// 0.1.4 - src/gpu_backend/cuda_q_std_prefill.rs", widened to the same page's batches
// of up to eight tokens.
//
// Why matrix cores. With a few tokens, a vector-ALU GEMV spends one f32 FMA per
// weight and token and reads x from LDS at T floats per weight; from about 3 tokens
// on those reads and FMAs, not the weight stream, set its time.
// v_mfma_f32_4x4x1_16b_f32 runs 16 independent 4 x 4 outer products per
// instruction: with the four A rows taken as four tokens and the four B columns as
// four weight rows, every lane block (four lanes) adds the products of one k, exact
// f32 operands in, f32 out, as the f32 leg asks (no reduced-precision inputs). Tokens
// come in groups of four (G = 1 or 2), so nothing is padded at T = 4 or 8.
//
// Work split. A workgroup has CW compute waves (4 or 12) and one wave that stages x.
// Compute wave w owns RQ row quads (for SwiGLU the first RQ/2 quads are gate rows and
// the rest the matching up rows) over the whole reduction, which the workgroup walks
// in rounds of 1024 k = 16 block pairs per row, one barrier per round. In a round,
// lane (b, q) (lane block b = lane / 4, q = lane % 4) holds pair b of weight row q of
// each quad, decoded exactly to f32 (w = d (u - c) with u the unsigned code: one
// conversion and one FMA), and x of token q (+ 4 g) at the same k: the pair's 64 k run
// through 64 instructions per quad and token group, each lane block adding its own k.
// x is read by the compute waves from LDS, where the staging wave stores each round
// in the order the lanes read it (double-buffered), so that the compute waves' own
// loads are weights only and waiting for one never waits for a younger x load.
//
// Loads. A compute wave reads its rows' round segments in coalesced 16-byte chunks
// into registers, DEPTH rounds ahead; a round's chunks go to the wave's LDS staging
// (double-buffered where that fits, else one buffer rewritten once the wave has read
// it) one round before it is computed, and each lane then takes the
// dwords of its pairs from there (a pair is 36 bytes for Q4_0, 68 for Q8_0, 4-byte
// aligned).
//
// Sums. Each lane block accumulates its k in the MFMA accumulators over all
// rounds; the 16 lane blocks are then added by a butterfly in a fixed order, so
// results do not vary between runs.
#include "pf_device.h"
#include "pf_internal.h"

namespace pf {

namespace {

template <int QT> struct MPair;
template <> struct MPair<Q4_0> {
    static constexpr int DW = 9;         // 36 bytes
    static constexpr int WORDS = 4;      // qs words per block, 8 weights each
    static constexpr float OFF = 8.0f;
};
template <> struct MPair<Q8_0> {
    static constexpr int DW = 17;        // 68 bytes
    static constexpr int WORDS = 8;      // qs words per block, 4 weights each
    static constexpr float OFF = 128.0f;
};

constexpr int RP = 16;             // pairs per row and round: one per lane block
constexpr int IN_FLIGHT_CHUNKS = 16;
constexpr int ROUND_K = 64 * RP;   // k per round

// One wave's weight chunks per round: 4 RQ rows of RP pairs.
template <int QT, int RQ> struct MStage {
    static constexpr int PB = MPair<QT>::DW * 4;        // bytes per pair
    static constexpr int ROW_CHUNKS = RP * PB / 16;     // 16-byte chunks per row segment
    static constexpr int CHUNKS = 4 * RQ * ROW_CHUNKS;
    static constexpr int NCH = (CHUNKS + 63) / 64;      // chunk loads per lane
    static constexpr int BYTES = NCH * 64 * 16;         // LDS bytes per wave
};

// x of one round in LDS, in float4 units: token group g, block h of the pair, float4
// f of the block (k = 32 h + 4 f .. + 3 of the pair), lane 4 b + q -> x[4 g + q][1024
// r + 64 b + 32 h + 4 f ..]. A wave's read of one (g, h, f) is 1 KB of consecutive
// bytes.
__device__ __forceinline__ int mx_index(int g, int h, int f, int l) { return ((g * 2 + h) * 8 + f) * 64 + l; }

// A workgroup has CW compute waves (4, or 12 where the weight has rows enough to give
// every CU 12 waves of one quad) and one more wave, index CW, that stages x.
// LDS: x of two rounds (double-buffered), then one or two weight staging buffers per
// compute wave (two where they fit).
template <int QT, int G, int RQ, int CW>
constexpr int mgemv_staging_buffers() { return 2 * G * 16384 + 2 * CW * MStage<QT, RQ>::BYTES <= 160 * 1024 ? 2 : 1; }
template <int QT, int G, int RQ, int CW>
constexpr int mgemv_lds_bytes() {
    return 2 * G * 16384 + mgemv_staging_buffers<QT, G, RQ, CW>() * CW * MStage<QT, RQ>::BYTES;
}

__device__ __forceinline__ float ubyte_f32(uint32_t w, int b) { return (float)((w >> (8 * b)) & 0xFFu); }

template <int QT, int EPI, int G, int RQ, int CW>
__global__ __launch_bounds__(64 * (CW + 1)) void gemv_mfma_kernel(const uint8_t *__restrict__ W,
                                                             const float *__restrict__ X,
                                                             float *__restrict__ Y, int n, int ldy,
                                                             int k, int T) {
    using PT = MPair<QT>;
    using ST = MStage<QT, RQ>;
    constexpr int NA = RQ * G < 2 ? 2 : 1;  // accumulator sets: independent MFMA chains
    constexpr int XF4 = 16 * G;             // x float4 the staging wave moves per lane and round
    // Rounds of weights in flight per compute wave: about IN_FLIGHT_CHUNKS 16-byte
    // loads per lane (three quarters of that with twelve compute waves, whose
    // registers are scarcer), from two to four rounds.
    constexpr int FLIGHT = CW == 4 ? IN_FLIGHT_CHUNKS : IN_FLIGHT_CHUNKS * 3 / 4;
    constexpr int DEPTH = FLIGHT / ST::NCH < 2 ? 2 : (FLIGHT / ST::NCH > 4 ? 4 : FLIGHT / ST::NCH);
    static_assert(EPI != EPI_SWIGLU || RQ % 2 == 0, "SwiGLU pairs gate and up quads");
    static_assert(mgemv_lds_bytes<QT, G, RQ, CW>() <= 160 * 1024, "LDS");

    __shared__ __attribute__((aligned(16))) uint8_t smem[mgemv_lds_bytes<QT, G, RQ, CW>()];
    f4_t *xl = reinterpret_cast<f4_t *>(smem);
    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lb = lane >> 2, q = lane & 3;

    const int npairs = k >> 6;
    const int rounds = (npairs + RP - 1) / RP;
    const int last_round = rounds - 1;
    // Rounds are padded to a multiple of DEPTH (the weight ring's slots are indexed
    // statically); a padded round only moves data. Every branch below depends on
    // the wave index, r and rounds alone: uniform over each wave, and the barriers
    // are reached by all waves the same number of times.
    const int padded = (rounds + DEPTH - 1) / DEPTH * DEPTH;

    if (wid == CW) {
        // The x stager: x of round r + 1 is requested at the start of round r and
        // stored to the other LDS buffer at its end. Token rows past T and k past the
        // row are read from clamped addresses instead of being zeroed: the sums of
        // tokens past T are never stored, and k past the row meets weights decoded
        // as exact zeros (their scale is taken as 0).
        f4_t xr[XF4];
        auto load_x = [&](int r) __attribute__((always_inline)) {
#pragma unroll
            for (int c = 0; c < XF4; ++c) {
                const int f = c & 7, h = (c >> 3) & 1, g = c >> 4;
                const int t = min(4 * g + q, T - 1);
                const int kk = ROUND_K * r + 64 * lb + 32 * h + 4 * f;
                xr[c] = *reinterpret_cast<const f4_t *>(X + (size_t)t * k + (kk < k ? kk : 0));
            }
        };
        auto store_x = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
            for (int c = 0; c < XF4; ++c) xl[buf * G * 1024 + 64 * c + lane] = xr[c];
        };
        load_x(0);
        store_x(0);
        __syncthreads();
        for (int r = 0; r < padded; ++r) {
            load_x(min(r + 1, last_round));
            store_x((r + 1) & 1);
            __syncthreads();
        }
        return;
    }

    constexpr int NSB = mgemv_staging_buffers<QT, G, RQ, CW>();
    uint8_t *wst = smem + 2 * G * 16384 + wid * (NSB * ST::BYTES);  // this wave's buffers
    const size_t row_bytes = (size_t)npairs * ST::PB;

    // Weight row of local row lr (quad lr / 4, row lr % 4) of this wave; rows past
    // the weight are clamped (their sums are never stored).
    constexpr int OUT_PER_WAVE = (EPI == EPI_SWIGLU) ? 2 * RQ : 4 * RQ;
    const int obase = (blockIdx.x * CW + wid) * OUT_PER_WAVE;
    auto weight_row = [&](int lr) __attribute__((always_inline)) {
        if constexpr (EPI == EPI_SWIGLU) {
            constexpr int HALF = 2 * RQ;  // gate rows of the wave
            const int o = min(obase + (lr % HALF), n - 1);
            return lr < HALF ? o : n + o;
        } else {
            return min(obase + lr, n - 1);
        }
    };

    // Per-lane chunk sources (fixed over the rounds except for the round offset).
    const uint8_t *csrc[ST::NCH];
    int cpos[ST::NCH];  // chunk index within its row segment
#pragma unroll
    for (int c = 0; c < ST::NCH; ++c) {
        const int j = min(lane + 64 * c, ST::CHUNKS - 1);
        const int lr = j / ST::ROW_CHUNKS;
        cpos[c] = j % ST::ROW_CHUNKS;
        csrc[c] = W + (size_t)weight_row(lr) * row_bytes;
    }
    // Ring of DEPTH rounds of weight chunks in registers: slot q % DEPTH holds round
    // q from DEPTH rounds before it is computed; during round q - 1 it goes to the
    // staging buffer q & 1 and the slot takes round q + DEPTH. Waiting for a slot
    // therefore never waits for a younger load.
    u4_t ch[DEPTH][ST::NCH];
    auto load_w = [&](int r, u4_t (&dst)[ST::NCH]) __attribute__((always_inline)) {
        const int np = min(RP, npairs - RP * r);
        const int last = np * ST::PB / 16 - 1;  // last chunk of the row segment this round
#pragma unroll
        for (int c = 0; c < ST::NCH; ++c)
            dst[c] = *reinterpret_cast<const u4_t *>(csrc[c] + (size_t)r * RP * ST::PB + 16 * min(cpos[c], last));
    };
    auto store_w = [&](const u4_t (&src)[ST::NCH], int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int c = 0; c < ST::NCH; ++c)
            *reinterpret_cast<u4_t *>(wst + buf * ST::BYTES + 16 * (lane + 64 * c)) = src[c];
    };

    f4_t acc[NA][RQ][G];
#pragma unroll
    for (int a = 0; a < NA; ++a)
#pragma unroll
        for (int p = 0; p < RQ; ++p)
#pragma unroll
            for (int g = 0; g < G; ++g) acc[a][p][g] = f4_t{0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int j = 0; j < DEPTH; ++j) load_w(min(j, last_round), ch[j]);
    store_w(ch[0], 0);
    load_w(min(DEPTH, last_round), ch[0]);
    __syncthreads();

    for (int r0 = 0; r0 < padded; r0 += DEPTH)
#pragma unroll
    for (int j = 0; j < DEPTH; ++j) {
        const int r = r0 + j;
        const int buf = r & 1;
        if (r < rounds) {
            // This lane's pair dwords, one set per quad.
            uint32_t dw[RQ][PT::DW];
#pragma unroll
            for (int p = 0; p < RQ; ++p) {
                const uint32_t *src = reinterpret_cast<const uint32_t *>(
                                          wst + (NSB == 2 ? buf : 0) * ST::BYTES + (4 * p + q) * (ST::ROW_CHUNKS * 16)) +
                                      PT::DW * lb;
#pragma unroll
                for (int i = 0; i < PT::DW; ++i) dw[p][i] = src[i];
            }
            const bool valid = RP * r + lb < npairs;
            const f4_t *xb_l = xl + buf * G * 1024;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                constexpr int MID = PT::DW / 2;  // dword holding block 1's scale (high half)
                // x of this block for the lane's token(s). With one compute wave per
                // SIMD all eight float4 are read at once, so that one wait covers
                // them; with three, per word (other waves cover the wait, and the
                // registers are scarcer).
                constexpr bool XB = CW == 4;
                f4_t xf[G][XB ? 8 : 1];
                if constexpr (XB) {
#pragma unroll
                    for (int g = 0; g < G; ++g)
#pragma unroll
                        for (int f = 0; f < 8; ++f) xf[g][f] = xb_l[mx_index(g, h, f, lane)];
                }
                float d[RQ], cd[RQ];
#pragma unroll
                for (int p = 0; p < RQ; ++p) {
                    const float sc = fp16_bits_to_f32(h == 0 ? (dw[p][0] & 0xFFFFu) : (dw[p][MID] >> 16));
                    d[p] = valid ? sc : 0.f;
                    cd[p] = -PT::OFF * d[p];  // exact: OFF is a power of two
                }
#pragma unroll
                for (int m = 0; m < PT::WORDS; ++m) {
                    // Q4_0 word m: k = 4m .. 4m+3 of the block (low nibbles), 16+4m ..
                    // (high nibbles); Q8_0 word m: k = 4m .. 4m+3.
                    f4_t xa[G], xh[G];
#pragma unroll
                    for (int g = 0; g < G; ++g) {
                        if constexpr (XB) {
                            xa[g] = xf[g][m];
                            if constexpr (QT == Q4_0) xh[g] = xf[g][4 + m];
                        } else {
                            xa[g] = xb_l[mx_index(g, h, m, lane)];
                            if constexpr (QT == Q4_0) xh[g] = xb_l[mx_index(g, h, 4 + m, lane)];
                        }
                    }
                    float wa[RQ][4], wb[RQ][4];
#pragma unroll
                    for (int p = 0; p < RQ; ++p) {
                        const uint32_t w = h == 0 ? __builtin_amdgcn_alignbyte(dw[p][m + 1], dw[p][m], 2)
                                                  : dw[p][MID + 1 + m];
                        if constexpr (QT == Q4_0) {
                            uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
                            // one v_cvt_f32_ubyteN per weight, no bit-field extract first
                            asm("" : "+v"(lo), "+v"(hi));
#pragma unroll
                            for (int c = 0; c < 4; ++c) {
                                wa[p][c] = fmaf(ubyte_f32(lo, c), d[p], cd[p]);
                                wb[p][c] = fmaf(ubyte_f32(hi, c), d[p], cd[p]);
                            }
                        } else {
                            const uint32_t u = w ^ 0x80808080u;
#pragma unroll
                            for (int c = 0; c < 4; ++c) wa[p][c] = fmaf(ubyte_f32(u, c), d[p], cd[p]);
                        }
                    }
                    // Consecutive instructions update different accumulators (quads and
                    // token groups innermost, or the two sets when there is one of each).
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        constexpr int SETS_PER_WORD = (QT == Q4_0) ? 2 : 1;
#pragma unroll
                        for (int e = 0; e < SETS_PER_WORD; ++e) {
                            const int a = NA == 2 ? (QT == Q4_0 ? e : c & 1) : 0;
#pragma unroll
                            for (int g = 0; g < G; ++g)
#pragma unroll
                                for (int p = 0; p < RQ; ++p)
                                    acc[a][p][g] = __builtin_amdgcn_mfma_f32_4x4x1f32(
                                        e == 0 ? xa[g][c] : xh[g][c], e == 0 ? wa[p][c] : wb[p][c],
                                        acc[a][p][g], 0, 0, 0);
                        }
                    }
                }
            }
        }
        // Round r + 1's weights to the other staging buffer (read last in round r - 1,
        // before the barrier that ended it), or with one buffer to the same one once
        // this wave's reads of it are done; the slot then takes round r + 1 + DEPTH.
        if constexpr (NSB == 2) {
            store_w(ch[(j + 1) % DEPTH], buf ^ 1);
        } else {
            wave_lds_sync();
            store_w(ch[(j + 1) % DEPTH], 0);
        }
        load_w(min(r + 1 + DEPTH, last_round), ch[(j + 1) % DEPTH]);
        __syncthreads();
    }

    // Lane (b, q), register i of acc[.][p][g] holds the sum over lane block b's k of
    // x[4 g + i] times weight row (p, q). Add the 16 lane blocks (lane bits 2..5).
    constexpr int NV = RQ * G * 4;
    float v[NV];
#pragma unroll
    for (int p = 0; p < RQ; ++p)
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float sum = acc[0][p][g][i];
                if constexpr (NA == 2) sum = sum + acc[1][p][g][i];
                v[(p * G + g) * 4 + i] = sum;
            }
#pragma unroll
    for (int dist = 4; dist < 64; dist <<= 1)
#pragma unroll
        for (int j = 0; j < NV; ++j) v[j] = v[j] + __shfl_xor(v[j], dist, 64);

    // Every lane now holds every sum; lane block b stores the values j with j % 16 == b.
    constexpr int PO = (EPI == EPI_SWIGLU) ? RQ / 2 : RQ;  // output quads
#pragma unroll
    for (int p = 0; p < PO; ++p)
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int j = (p * G + g) * 4 + i;
                const int t = 4 * g + i;
                const int o = obase + 4 * p + q;
                if (j % 16 != lb || t >= T || o >= n) continue;
                float y = v[j];
                if constexpr (EPI == EPI_SWIGLU) y = silu_f32(y) * v[((p + RQ / 2) * G + g) * 4 + i];
                float *dst = Y + (size_t)t * ldy + o;
                if constexpr (EPI == EPI_RESIDUAL)
                    *dst = *dst + y;
                else
                    *dst = y;
            }
}

template <int QT, int EPI, int G, int RQ, int CW>
hipError_t launch_mq(const GemmArgs &a, hipStream_t s) {
    constexpr int OUT_PER_WG = CW * ((EPI == EPI_SWIGLU) ? 2 * RQ : 4 * RQ);
    const int blocks = (a.n + OUT_PER_WG - 1) / OUT_PER_WG;
    hipLaunchKernelGGL((gemv_mfma_kernel<QT, EPI, G, RQ, CW>), dim3(blocks), dim3(64 * (CW + 1)), 0, s, a.W, a.X,
                       a.Y, a.n, a.ldy, a.k, a.T);
    return hipGetLastError();
}

// A form fits when its LDS does and its registers do: a Q8_0 pair is 17 dwords per
// quad, so Q8_0 takes at most two quads per wave with four compute waves and one with
// twelve (more spilled to scratch).
template <int QT, int G, int RQ, int CW>
constexpr bool mgemv_fits() {
    return mgemv_lds_bytes<QT, G, RQ, CW>() <= 160 * 1024 && (QT == Q4_0 || RQ * (CW == 12 ? 2 : 1) <= 2);
}

// Waves and row quads per workgroup: twelve compute waves of one quad (SwiGLU: of a
// gate and an up quad) where that fits in LDS and still gives every CU a workgroup
// (three waves per SIMD cover each other's waits); else four compute waves with two
// quads each (SwiGLU: four, the gate and up quads of two), or one where two would
// leave CUs without a workgroup.
template <int QT, int EPI, int G>
hipError_t launch_mg(const GemmArgs &a, hipStream_t s) {
    constexpr int CUS = 256;
    constexpr int PER = (EPI == EPI_SWIGLU ? 2 : 4);  // outputs per wave and row quad
    auto enough = [&](int cw, int rq) { return (a.n + cw * PER * rq - 1) / (cw * PER * rq) >= CUS; };
    if constexpr (EPI == EPI_SWIGLU) {
        if constexpr (mgemv_fits<QT, G, 2, 12>())
            if (enough(12, 2)) return launch_mq<QT, EPI, G, 2, 12>(a, s);
        if constexpr (mgemv_fits<QT, G, 4, 4>())
            if (enough(4, 4)) return launch_mq<QT, EPI, G, 4, 4>(a, s);
        return launch_mq<QT, EPI, G, 2, 4>(a, s);
    } else {
        if constexpr (mgemv_fits<QT, G, 1, 12>())
            if (enough(12, 1)) return launch_mq<QT, EPI, G, 1, 12>(a, s);
        if (enough(4, 2)) return launch_mq<QT, EPI, G, 2, 4>(a, s);
        return launch_mq<QT, EPI, G, 1, 4>(a, s);
    }
}

template <int QT, int EPI>
hipError_t launch_me(const GemmArgs &a, hipStream_t s) {
    return a.T <= 4 ? launch_mg<QT, EPI, 1>(a, s) : launch_mg<QT, EPI, 2>(a, s);
}

template <int QT>
hipError_t launch_mqt(const GemmArgs &a, hipStream_t s) {
    switch (a.epilogue) {
    case EPI_PLAIN: return launch_me<QT, EPI_PLAIN>(a, s);
    case EPI_RESIDUAL: return launch_me<QT, EPI_RESIDUAL>(a, s);
    default: return launch_me<QT, EPI_SWIGLU>(a, s);
    }
}

}  // namespace

hipError_t launch_gemv_mfma(const GemmArgs &a, hipStream_t s) {
    // 1 <= T <= 8 is checked by the API.
    return a.qtype == Q4_0 ? launch_mqt<Q4_0>(a, s) : launch_mqt<Q8_0>(a, s);
}

}  // namespace pf
