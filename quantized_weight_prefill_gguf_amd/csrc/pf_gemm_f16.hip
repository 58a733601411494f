// Tiled GEMM, f16 leg: fp16 inputs, fp32 accumulation, f32 output
// (v_mfma_f32_32x32x16_f16), the f16 leg of the page "aprender-serve 0.70.2 -
// src/cuda/executor/gdn_prefill_ops.rs" (module doc, group 1, and
// `qwen35_project_rows_f16`): weights and activations rounded to fp16,
// accumulation and output in fp32. Unlike that page nothing is cached or
// converted in HBM: X is rounded to fp16 while it is staged into LDS, and each
// weight block is decoded to fp16 in registers right before the MFMAs that eat it.
//
// Workgroup: 256 threads = 4 waves in a 2 x 2 grid; tile MT token rows x NW weight
// rows; each wave owns (MT/2) x (NW/2) fp32 accumulators as 32 x 32 MFMA tiles.
// K loop: one 32-weight block per step = two 32x32x16 MFMAs per tile.
//  - Weight bytes move in chunks of 8 blocks (256 k): a row's chunk is 144 (Q4_0)
//    or 272 (Q8_0) bytes, 16-byte aligned in HBM when k % 256 == 0, so it is copied
//    raw (GGUF AoS as stored) with 16-byte loads into a double-buffered LDS chunk,
//    1/8 of the next chunk per step.
//  - X moves one step (32 k) at a time: f32 loads, RNE to fp16, stored in LDS in
//    the k order the weight decode produces, two steps ahead of its use.
//  - Software pipeline: while step s's MFMAs run, the wave reads step s+1's A
//    fragments and raw weight words from LDS and decodes the weights, so neither
//    LDS latency nor the decode sits between barrier and matrix core.
//  - The 8 steps of a chunk are unrolled, so every LDS offset and the alignment
//    of every block inside the chunk are compile-time constants.
// Lane (c, h) of a B fragment (column c, half h) decodes 16 weights of its
// column's block: Q4_0 qs bytes 8h .. 8h+7 (low nibbles feed the first MFMA, high
// nibbles the second), Q8_0 int8 bytes 8h .. 8h+7 and 16+8h .. 16+8h+7.
//
// GATE_UP_SWIGLU: each 32-column tile holds 16 gate rows and the 16 up rows of
// the same outputs, so g and u of one output sit in lanes c and c+16 of the same
// register; the epilogue swaps them across the two lane groups.
//
// Large-n shapes run one workgroup per output tile. With a caller workspace, narrow
// ones (n = 4096 at T = 512) and short chunks split K over workgroups that store
// their partial sums in the workspace; a second kernel adds them in split order, so
// the result is the same from run to run. Without a workspace nothing splits.
#include <type_traits>

#include "pf_device.h"
#include "pf_internal.h"

namespace pf {

namespace {

template <int QT> struct ChunkTraits {
    static constexpr int BB = BlockTraits<QT>::BYTES;
    static constexpr int ROW = 8 * BB;      // bytes of one row's chunk (144 / 272)
    static constexpr int U4 = ROW / 16;     // 16-byte pieces per row chunk (9 / 17)
};
// Further types on the cooperative kernel: a row's 256-k chunk is one super-block
// (Q4_K 144 bytes, Q5_K 176) or eight F16 groups (512 bytes), every one a whole
// number of 16-byte pieces, 16-byte aligned. BB (a 32-weight block) has no meaning.
template <> struct ChunkTraits<XQ_Q4_K> {
    static constexpr int BB = 0, ROW = 144, U4 = 9;
};
template <> struct ChunkTraits<XQ_Q5_K> {
    static constexpr int BB = 0, ROW = 176, U4 = 11;
};
template <> struct ChunkTraits<XQ_F16> {
    static constexpr int BB = 0, ROW = 512, U4 = 32;
};
// IQ4_XS: 136 bytes per super-block, 8-byte aligned only: staged in 8-byte pieces
// (U4 counts pieces of PIECE bytes).
template <> struct ChunkTraits<XQ_IQ4_XS> {
    static constexpr int BB = 0, ROW = 136, U4 = 17, PIECE = 8;
};
// Q6_K: 210 bytes per super-block, 2-byte aligned. With rows a multiple of 4 bytes
// (k % 512 == 0) a chunk starts sh = 2 (c % 2) bytes past a dword boundary, the same
// for every row: a row's LDS chunk (216 bytes) holds the bytes from that boundary, as
// 26 pieces of 8 bytes and a 27th whose first dword is chunk bytes 208 - sh .. 211 - sh,
// read as two halfwords so that no load passes the chunk's end. GROW: bytes per row
// chunk in the weight (ROW is the LDS row).
template <> struct ChunkTraits<XQ_Q6_K> {
    static constexpr int BB = 0, ROW = 216, U4 = 27, PIECE = 8, GROW = 210;
};
template <int QT> constexpr int chunk_piece() {
    if constexpr (QT == XQ_IQ4_XS || QT == XQ_Q6_K) return ChunkTraits<QT>::PIECE;
    else return 16;
}
template <int QT> constexpr int chunk_grow() {
    if constexpr (QT == XQ_Q6_K) return ChunkTraits<QT>::GROW;
    else return ChunkTraits<QT>::ROW;
}
template <int QT> constexpr bool coop_xq() {
    return QT == XQ_Q4_K || QT == XQ_Q5_K || QT == XQ_F16 || QT == XQ_IQ4_XS || QT == XQ_Q6_K;
}
typedef uint32_t u2a4_t __attribute__((ext_vector_type(2), aligned(4)));  // 4-byte aligned

// Sub-block j's 6-bit scale and min of a Q4_K / Q5_K super-block header (d, dmin, then
// the 12 scale bytes): j < 4 take the low 6 bits of bytes j and j + 4; j >= 4 the
// nibbles of byte j + 4 with the top 2 bits of bytes j - 4 (scale) and j (min).
template <int J>
__device__ __forceinline__ void kq_scale_min(const u4_t &hdr, uint32_t &sc, uint32_t &mn) {
    auto sb = [&](int i) { return (hdr[(4 + i) >> 2] >> (8 * ((4 + i) & 3))) & 0xFFu; };
    if constexpr (J < 4) {
        sc = sb(J) & 63u;
        mn = sb(J + 4) & 63u;
    } else {
        sc = (sb(J + 4) & 15u) | ((sb(J - 4) >> 6) << 4);
        mn = (sb(J + 4) >> 4) | ((sb(J) >> 6) << 4);
    }
}

typedef float f16v_t __attribute__((ext_vector_type(16)));

// Staged X: within each group of four k, Q4_0 fragments take the order 0, 2, 1, 3
// (the nibble-pair order of q4_word_decode); Q8_0 takes natural order. Lane half
// h of MFMA s reads halves 16s + 8h .. 16s + 8h + 7 of the row's block segment.
template <int QT> __device__ __forceinline__ u2_t x_pack(f4_t v) {
    if constexpr (QT == Q4_0)
        return u2_t{h2_bits(h2_t{(_Float16)v[0], (_Float16)v[2]}),
                    h2_bits(h2_t{(_Float16)v[1], (_Float16)v[3]})};
    else
        return u2_t{h2_bits(h2_t{(_Float16)v[0], (_Float16)v[1]}),
                    h2_bits(h2_t{(_Float16)v[2], (_Float16)v[3]})};
}

}  // namespace

// Up to this many token rows the GEMM below 256 rows takes one row tile.
constexpr int SHORT_T = 128;
// Workgroups of a one-row-of-waves tile (MT x 128, waves 1 x 4) resident per CU
// (waves per SIMD), as its LDS (Q4_0: 41 KB at 32 rows, 45 KB at 64, 53 KB at 128;
// Q8_0: 74 KB and up; Q4_K / Q5_K / IQ4_XS: 41 / 49 / 39 KB at 32 rows) and registers
// allow. Three at 32 rows hold the further types in 148-164 registers: gate/up 2 x
// 12288 x 4096 at T = 16 took 30-33 us against 34-39 with two (the down projection
// 4096 x 12288 gave up 0.5-1 us to its larger split).
constexpr int short_tile_waves(int qt, int mt) {
    return mt > 64 ? 1 : ((qt == Q4_0 || qt == XQ_Q4_K || qt == XQ_Q5_K || qt == XQ_IQ4_XS) && mt <= 32) ? 3 : 2;
}

// Global weight row of local tile row lr, or -1 past the weight.
template <int EPI, int NW>
__device__ __forceinline__ int f16_weight_row(int tile_n, int lr, int n) {
    if constexpr (EPI == EPI_SWIGLU) {
        // 32-row groups: rows 0..15 gate, 16..31 up, for 16 consecutive outputs
        const int o = tile_n * (NW / 2) + (lr >> 5) * 16 + (lr & 15);
        if (o >= n) return -1;
        return (lr & 16) ? n + o : o;
    } else {
        const int r = tile_n * NW + lr;
        return r < n ? r : -1;
    }
}

template <int QT, int EPI, int MT, int NW, bool SPLIT, bool XH, bool ROW1>
__global__ __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(1, ROW1 ? short_tile_waves(QT, MT) : 1)))
void gemm_f16_kernel(const uint8_t *__restrict__ W, const void *__restrict__ Xv,
                     float *__restrict__ Y, int n, int ldy, int k, int T, int tiles_m, int tiles_n,
                     int splits, long pstride) {
    using CT = ChunkTraits<QT>;
    constexpr int BB = CT::BB;
    // Further types (Q4_K, Q5_K, IQ4_XS, Q6_K with k % 512 == 0): a row's 256-k chunk is
    // one super-block, and step blk its sub-block blk.
    constexpr bool XQ = coop_xq<QT>();
    static_assert(!XQ || QT != XQ_F16, "further types: not F16");
    // Waves: WVM x WVN over the tile. ROW1 tiles (few token rows) put all four side
    // by side along the weight rows, so that no two decode the same columns.
    constexpr int WVM = ROW1 ? 1 : 2;
    constexpr int WVN = 4 / WVM;
    constexpr int IT = MT / (32 * WVM);   // 32-row MFMA tiles per wave
    constexpr int JT = NW / (32 * WVN);   // 32-column MFMA tiles per wave
    static_assert(IT >= 1 && JT >= 1 && MT % 32 == 0, "tile shape");
    constexpr int XF4 = MT / 32;          // f32 X: float4 loads per thread per step
    constexpr int XH4 = MT >= 64 ? MT / 64 : 1;  // fp16 X: 16-byte loads per thread per step
    // fp16 X staging covers 64 rows per pass; a 32-row tile uses threads < 128 only.
    const bool xh_store = MT >= 64 || threadIdx.x < 128;
    constexpr int U4 = CT::U4;                      // pieces per row chunk
    constexpr int PIECE = chunk_piece<QT>();        // bytes per piece (16; IQ4_XS 8)
    constexpr int WROW = CT::ROW;
    constexpr int WBUF = NW * WROW + 16;            // +16: decode reads a dword past a row
    constexpr int NW32 = (QT == Q4_0) ? 2 : 4;      // qs words per lane per block
    constexpr int GROW = chunk_grow<QT>();          // bytes per row chunk in the weight
    // a piece in flight: 16 bytes, 8 (IQ4_XS), or Q6_K's 8 and two halfwords
    typedef typename std::conditional<PIECE == 16 || QT == XQ_Q6_K, u4_t, u2_t>::type piece_t;

    // One LDS block: the K loop's two X buffers and two weight chunks; after the
    // loop, the SwiGLU epilogue reuses its start as 4 per-wave 32 x 36 float slots.
    constexpr int XBUF_BYTES = MT * 32 * 2;
    constexpr int LOOP_BYTES = 2 * XBUF_BYTES + 2 * WBUF;
    constexpr int EPI_BYTES = 4 * 32 * 36 * 4;
    __shared__ __attribute__((aligned(16))) uint8_t smem[LOOP_BYTES > EPI_BYTES ? LOOP_BYTES : EPI_BYTES];
    _Float16 (*xs)[MT * 32] = reinterpret_cast<_Float16 (*)[MT * 32]>(smem);
    uint8_t (*wsm)[WBUF] = reinterpret_cast<uint8_t (*)[WBUF]>(smem + 2 * XBUF_BYTES);
    static_assert(WBUF % 16 == 0 && XBUF_BYTES % 16 == 0, "LDS carve-up keeps 16-byte alignment");

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WVN, wn = wave % WVN;
    const int c = lane & 31, h = lane >> 5;

    // Workgroup -> tile. Dispatch spreads consecutive workgroup ids over the 8
    // XCDs; remap so that each XCD gets a contiguous run of tiles in which the M
    // tiles of one weight tile are adjacent (they share its chunks in that L2).
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
    const int nch = c_end - c_begin;
    if (nch <= 0) return;  // cannot happen (splits <= chunks); keeps the loop simple
    const int nsteps = 8 * nch;
    const uint32_t row_bytes = XQ ? (uint32_t)(k >> 8) * GROW : (uint32_t)(k >> 5) * BB;

    // ---- staging assignments (fixed over the K loop), as 32-bit byte offsets
    // from uniform bases. Global loads are all unconditional so that the wait
    // counters stay exact: rows past T or past the weight read a valid row
    // instead; such rows only feed outputs that are never stored.
    // Staged X rows are 32 halves (4 chunks of 16 bytes); chunk q of row r sits at
    // chunk q ^ ((r >> 2) & 3), which keeps both the staging writes and the
    // fragment reads free of LDS bank conflicts.
    // f32 X (XH false): thread t converts float4 (t & 7) of rows (t >> 3) + 32 i.
    // fp16 X (XH true, already in fragment k order): thread t copies 16-byte chunk
    // (t & 3) of rows (t >> 2) + 64 i.
    // Byte offsets: fp16 X holds T k < 2^31 halves, so 2 t k stays below 2^32; f32
    // X reaches 4 t k >= 2^32 once t k >= 2^30, so its offsets are 64-bit.
    constexpr int XN = XH ? XH4 : XF4;
    const uint8_t *xbase = reinterpret_cast<const uint8_t *>(Xv) + (size_t)c_begin * 256 * (XH ? 2 : 4);
    typedef typename std::conditional<XH, uint32_t, uint64_t>::type xoff_t;
    xoff_t xoff[XN];
    int xdst;
    if constexpr (XH) {
#pragma unroll
        for (int i = 0; i < XN; ++i) {
            const int t = min(m0 + (tid >> 2) + 64 * i, T - 1);
            xoff[i] = ((uint32_t)t * (uint32_t)k + 8 * (tid & 3)) * 2;
        }
        // rows (tid >> 2) + 64 i share (row >> 2) & 3
        xdst = (tid >> 2) * 32 + (((tid & 3) ^ ((tid >> 4) & 3)) << 3);
    } else {
#pragma unroll
        for (int i = 0; i < XN; ++i) {
            const int t = min(m0 + (tid >> 3) + 32 * i, T - 1);
            xoff[i] = ((uint64_t)t * (uint64_t)k + 4 * (tid & 7)) * 4;
        }
        // rows (tid >> 3) + 32 i share (row >> 2) & 3
        xdst = (tid >> 3) * 32 + ((((tid & 7) >> 1) ^ ((tid >> 5) & 3)) << 3) + 4 * (tid & 1);
    }
    // Weight staging. Slice S of a chunk is its rows S RS .. S RS + RS - 1 (RS = NW
    // / 8), whole: RS * U4 pieces (16 bytes, IQ4_XS and Q6_K 8), which the threads take in
    // order, piece f = tid + 256 i being piece f % U4 of slice row f / U4. Consecutive
    // lanes thus read consecutive bytes of a row. Since RS * U4 is the same for every
    // slice, a thread's (row in slice, piece) is fixed; only the weight row of slice row
    // rr, i.e. its global offset, depends on S.
    // Q6_K (210-byte super-blocks, rows a multiple of 4 bytes): chunk c starts sh = 2 (c
    // % 2) bytes past a dword boundary in every row, and its 216-byte LDS row holds the
    // bytes from that boundary: pieces 0 .. 25 are 8-byte loads from there, and the 27th
    // (chunk bytes 208 - sh .. 211 - sh) is assembled from two halfword loads when stored,
    // so that no load passes the chunk's end.
    constexpr int RS = NW / 8;
    constexpr int SP = RS * U4;                      // pieces per slice
    constexpr int NPT = (SP + 255) / 256;            // pieces per thread per slice
    uint32_t wsrc[8][NPT];                           // [slice][piece]: row offset + piece
    int wdst[NPT];                                   // LDS offset within slice 0
    bool wvalid[NPT];
    int wpo[NPT];                                    // Q6_K: the piece's offset past the boundary
    bool wlast[NPT];                                 // Q6_K: the 27th piece
    const uint8_t *wbase = W + (size_t)c_begin * GROW;
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
        const int f = tid + 256 * i;
        wvalid[i] = f < SP;
        const int ff = wvalid[i] ? f : 0;
        const int rr = ff / U4, pp = ff % U4;
        wdst[i] = rr * WROW + PIECE * pp;
        wlast[i] = pp == U4 - 1;
        wpo[i] = wlast[i] ? 200 : PIECE * pp;
#pragma unroll
        for (int S = 0; S < 8; ++S) {
            int gr = f16_weight_row<EPI, NW>(tn, S * RS + rr, n);
            gr = gr < 0 ? 0 : gr;
            wsrc[S][i] = (uint32_t)gr * row_bytes + (QT == XQ_Q6_K ? 0 : PIECE * pp);
        }
    }

    // LDS offsets of this lane's B rows (column c of tile j: bbase + j 32 WROW) and
    // A fragments.
    const int bbase = (wn * JT * 32 + c) * WROW;
    const int sw = (c >> 2) & 3;
    const int arow = (wm * IT * 32 + c) * 32;
    const int aoff[2] = {arow + ((h ^ sw) << 3), arow + (((2 + h) ^ sw) << 3)};

    f16v_t acc[IT][JT];
#pragma unroll
    for (int i = 0; i < IT; ++i)
#pragma unroll
        for (int j = 0; j < JT; ++j) acc[i][j] = f16v_t{};

    h8_t afr[2][IT][2];   // A fragments [step parity][tile][MFMA half]
    h8_t bfr[2][JT][2];   // decoded B fragments [step parity][tile][MFMA half]
    // Staging loads run PD steps ahead of their LDS writes (a ring of PD register
    // sets): under a full weight stream the HBM latency exceeds two steps, and the
    // wait counters complete loads in order.
    constexpr int PD = 4;
    f4_t xr[XF4];         // f32 X for the staging write of the next step
    u4_t xh[PD][XH4];     // fp16 X for the staging writes of the next PD steps
    piece_t wr[PD][NPT];  // weight slices for the writes of the next PD steps

    auto load_a = [&](int xb, h8_t (&dst)[IT][2]) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < IT; ++i)
#pragma unroll
            for (int s = 0; s < 2; ++s)
                dst[i][s] = *reinterpret_cast<const h8_t *>(&xs[xb][aoff[s] + i * 32 * 32]);
    };
    // This lane's raw bytes of block `blk` (compile-time) for its JT B columns: the
    // scale and the aligned dwords that hold its qs words (NRAW of them; when the
    // qs start 2 bytes into a dword, a word straddles two dwords).
    // Further types: the header dwords (Q4_K / Q5_K: d, dmin and the 12 scale bytes;
    // IQ4_XS: d, scales_h, scales_l), then the dwords of codes for k = 8 h .. 8 h + 7
    // and 16 + 8 h .. 16 + 8 h + 7 of sub-block blk (Q4_K / Q5_K: the qs bytes, nibble
    // half blk % 2; IQ4_XS: one 8-byte run whose low nibbles are the first eight and
    // high nibbles the second), and for Q5_K the qh dwords of the same k.
    // Q6_K (sub-block blk = 4 H + C): its ql bytes 64 H + 32 (C % 2) + 8 h .. and 16 bytes
    // on, and its qh bytes 128 + 32 H + 8 h .. and 16 on, each 8-byte run as the three
    // dwords around it (the chunk sits sh bytes into its LDS row); then the halfword of the
    // two scales (bytes 192 + 8 H + 2 C and one on: l < 16 and l >= 16), d, and sh.
    constexpr int NRAW = QT == XQ_Q6_K ? 15 : QT == XQ_Q5_K ? 12 : QT == XQ_Q4_K ? 8 : QT == XQ_IQ4_XS ? 4
                                                                                   : (QT == Q4_0) ? 3 : 6;
    auto read_b = [&](int wbuf, auto blk_c, uint32_t (&d16)[JT], uint32_t (&raw)[JT][NRAW])
        __attribute__((always_inline)) {
        constexpr int blk = decltype(blk_c)::value;
        constexpr int SH = (blk * BB + 2) & 3;
        const uint8_t *wb = wsm[wbuf];
        if constexpr (XQ) {
            (void)d16;
#pragma unroll
            for (int j = 0; j < JT; ++j) {
                const uint8_t *rb = wb + bbase + j * 32 * WROW;  // the column's super-block
                if constexpr (QT == XQ_Q6_K) {
                    constexpr int H = blk >> 2, C = blk & 3;
                    const uint32_t sh = ((c_begin ^ wbuf) & 1) * 2;
                    auto run = [&](int off, int at) __attribute__((always_inline)) {
                        const u2_t a = *reinterpret_cast<const u2_t *>(rb + off);
                        raw[j][at] = a[0];
                        raw[j][at + 1] = a[1];
                        raw[j][at + 2] = *reinterpret_cast<const uint32_t *>(rb + off + 8);
                    };
                    run(64 * H + 32 * (C & 1) + 8 * h, 0);
                    run(64 * H + 32 * (C & 1) + 16 + 8 * h, 3);
                    run(128 + 32 * H + 8 * h, 6);
                    run(128 + 32 * H + 16 + 8 * h, 9);
                    raw[j][12] = *reinterpret_cast<const uint16_t *>(rb + sh + 192 + 8 * H + 2 * C);
                    raw[j][13] = *reinterpret_cast<const uint16_t *>(rb + sh + 208);
                    raw[j][14] = sh;
                } else if constexpr (QT == XQ_IQ4_XS) {
                    const u2_t hd = *reinterpret_cast<const u2_t *>(rb);
                    const u2_t cw = *reinterpret_cast<const u2_t *>(rb + 8 + 16 * blk + 8 * h);
                    raw[j][0] = hd[0]; raw[j][1] = hd[1];
                    raw[j][2] = cw[0]; raw[j][3] = cw[1];
                } else {
                    constexpr int QS = QT == XQ_Q5_K ? 48 : 16;  // qs offset in the super-block
                    const u4_t hd = *reinterpret_cast<const u4_t *>(rb);
                    const u2_t q0 = *reinterpret_cast<const u2_t *>(rb + QS + 32 * (blk >> 1) + 8 * h);
                    const u2_t q1 = *reinterpret_cast<const u2_t *>(rb + QS + 32 * (blk >> 1) + 16 + 8 * h);
#pragma unroll
                    for (int e = 0; e < 4; ++e) raw[j][e] = hd[e];
                    raw[j][4] = q0[0]; raw[j][5] = q0[1];
                    raw[j][6] = q1[0]; raw[j][7] = q1[1];
                    if constexpr (QT == XQ_Q5_K) {
                        const u2_t h0 = *reinterpret_cast<const u2_t *>(rb + 16 + 8 * h);
                        const u2_t h1 = *reinterpret_cast<const u2_t *>(rb + 32 + 8 * h);
                        raw[j][8] = h0[0]; raw[j][9] = h0[1];
                        raw[j][10] = h1[0]; raw[j][11] = h1[1];
                    }
                }
            }
        } else {
#pragma unroll
            for (int j = 0; j < JT; ++j) {
                const int base = bbase + j * 32 * WROW + blk * BB;
                d16[j] = *reinterpret_cast<const uint16_t *>(wb + base);
                const uint32_t *al = reinterpret_cast<const uint32_t *>(wb + base + 2 + 8 * h - SH);
                if constexpr (SH == 0) {
#pragma unroll
                    for (int w = 0; w < NW32; ++w) raw[j][w] = al[(w & 1) + 4 * (w >> 1)];
                } else {
#pragma unroll
                    for (int g = 0; g < NW32 / 2; ++g)
#pragma unroll
                        for (int e = 0; e < 3; ++e) raw[j][3 * g + e] = al[4 * g + e];
                }
            }
        }
    };
    // Decode raw bytes read by read_b for block `blk` into the B fragments.
    auto decode_b = [&](auto blk_c, const uint32_t (&d16)[JT], const uint32_t (&raw)[JT][NRAW],
                        h8_t (&dst)[JT][2]) __attribute__((always_inline)) {
        constexpr int blk = decltype(blk_c)::value;
        constexpr int SH = (blk * BB + 2) & 3;
        if constexpr (XQ) {
            // Each weight's f32 value as the further types define it, made opaque, then
            // binary16 (RNE): Q4_K / Q5_K (d s) q - dmin m as one FMA ((d s) q is exact,
            // so it rounds once, as the subtraction would); IQ4_XS d (ls - 32) grid,
            // exact in f32.
            (void)d16;
#pragma unroll
            for (int j = 0; j < JT; ++j) {
                uint32_t p[8];
                if constexpr (QT == XQ_Q6_K) {
                    // (d sc) (q - 32): d sc is exact, the product rounds once in f32. q: 4
                    // low bits from ql (high nibble for C >= 2), 2 high bits from qh bits
                    // 2 C, 2 C + 1.
                    constexpr int C = blk & 3;
                    const uint32_t sh = raw[j][14];
                    auto al = [&](int a) __attribute__((always_inline)) {
                        return __builtin_amdgcn_alignbyte(raw[j][a + 1], raw[j][a], sh);
                    };
                    const uint32_t ql[4] = {al(0), al(1), al(3), al(4)};
                    const uint32_t qh[4] = {al(6), al(7), al(9), al(10)};
                    const float d = fp16_bits_to_f32(raw[j][13]);
                    const float ds[2] = {d * (float)(int8_t)(uint8_t)(raw[j][12] & 0xFFu),
                                         d * (float)(int8_t)(uint8_t)(raw[j][12] >> 8)};
#pragma unroll
                    for (int w = 0; w < 4; ++w) {
                        const uint32_t q = ((ql[w] >> (4 * (C >> 1))) & 0x0F0F0F0Fu) |
                                           (((qh[w] >> (2 * C)) & 0x03030303u) << 4);
                        float v[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            v[e] = ds[w >> 1] * (float)((int)((q >> (8 * e)) & 0xFFu) - 32);
                            asm("" : "+v"(v[e]));
                        }
                        p[2 * w] = h2_bits(h2_t{(_Float16)v[0], (_Float16)v[1]});
                        p[2 * w + 1] = h2_bits(h2_t{(_Float16)v[2], (_Float16)v[3]});
                    }
                } else if constexpr (QT == XQ_IQ4_XS) {
                    const uint32_t h0 = raw[j][0], sl = raw[j][1];
                    const uint32_t ls = ((sl >> (4 * blk)) & 15u) | (((h0 >> (16 + 2 * blk)) & 3u) << 4);
                    const float dl = fp16_bits_to_f32(h0 & 0xFFFFu) * (float)((int)ls - 32);
#pragma unroll
                    for (int w = 0; w < 4; ++w) {
                        const uint32_t g = iq4_grid_bytes((raw[j][2 + (w & 1)] >> (4 * (w >> 1))) & 0x0F0F0F0Fu);
                        float v[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            v[e] = dl * (float)(int8_t)(uint8_t)(g >> (8 * e));
                            asm("" : "+v"(v[e]));
                        }
                        p[2 * w] = h2_bits(h2_t{(_Float16)v[0], (_Float16)v[1]});
                        p[2 * w + 1] = h2_bits(h2_t{(_Float16)v[2], (_Float16)v[3]});
                    }
                } else {
                    uint32_t sc, mn;
                    kq_scale_min<blk>(u4_t{raw[j][0], raw[j][1], raw[j][2], raw[j][3]}, sc, mn);
                    const float a = fp16_bits_to_f32(raw[j][0] & 0xFFFFu) * (float)sc;
                    const float b = fp16_bits_to_f32(raw[j][0] >> 16) * (float)mn;
#pragma unroll
                    for (int w = 0; w < 4; ++w) {
                        uint32_t q = (raw[j][4 + w] >> (4 * (blk & 1))) & 0x0F0F0F0Fu;
                        if constexpr (QT == XQ_Q5_K) q |= ((raw[j][8 + w] >> blk) & 0x01010101u) << 4;
                        float v[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            v[e] = fmaf(a, (float)((q >> (8 * e)) & 0xFFu), -b);
                            asm("" : "+v"(v[e]));
                        }
                        p[2 * w] = h2_bits(h2_t{(_Float16)v[0], (_Float16)v[1]});
                        p[2 * w + 1] = h2_bits(h2_t{(_Float16)v[2], (_Float16)v[3]});
                    }
                }
                dst[j][0] = __builtin_bit_cast(h8_t, u4_t{p[0], p[1], p[2], p[3]});
                dst[j][1] = __builtin_bit_cast(h8_t, u4_t{p[4], p[5], p[6], p[7]});
            }
        } else {
#pragma unroll
            for (int j = 0; j < JT; ++j) {
                uint32_t q[NW32];
#pragma unroll
                for (int w = 0; w < NW32; ++w) {
                    if constexpr (SH == 0)
                        q[w] = raw[j][w];
                    else
                        q[w] = __builtin_amdgcn_alignbyte(raw[j][3 * (w >> 1) + (w & 1) + 1],
                                                          raw[j][3 * (w >> 1) + (w & 1)], SH);
                }
                const h2_t d2 = as_h2(d16[j] | (d16[j] << 16));
                uint32_t p[8];
                if constexpr (QT == Q4_0) {
                    q4_word_decode(q[0], d2, p[0], p[1], p[4], p[5]);
                    q4_word_decode(q[1], d2, p[2], p[3], p[6], p[7]);
                } else {
                    q8_word_to_h4(q[0], d2, p + 0);
                    q8_word_to_h4(q[1], d2, p + 2);
                    q8_word_to_h4(q[2], d2, p + 4);
                    q8_word_to_h4(q[3], d2, p + 6);
                }
                dst[j][0] = __builtin_bit_cast(h8_t, u4_t{p[0], p[1], p[2], p[3]});
                dst[j][1] = __builtin_bit_cast(h8_t, u4_t{p[4], p[5], p[6], p[7]});
            }
        }
    };
    // f32 X: registers (one step ahead) -> fp16 in LDS.
    auto store_x = [&](int xb) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < XF4; ++i)
            *reinterpret_cast<u2_t *>(&xs[xb][xdst + i * 32 * 32]) = x_pack<QT>(xr[i]);
    };
    auto fetch_x = [&](int step) __attribute__((always_inline)) {
        const uint8_t *xb = xbase + 128 * min(step, nsteps - 1);
#pragma unroll
        for (int i = 0; i < XF4; ++i) xr[i] = *reinterpret_cast<const f4_t *>(xb + xoff[i]);
    };
    // fp16 X: registers (two steps ahead) -> LDS, no conversion.
    auto store_xh = [&](int xb, const u4_t (&src)[XH4]) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < XH4; ++i)
            if (xh_store) *reinterpret_cast<u4_t *>(&xs[xb][xdst + i * 64 * 32]) = src[i];
    };
    auto fetch_xh = [&](int step, u4_t (&dst)[XH4]) __attribute__((always_inline)) {
        const uint8_t *xb = xbase + 64 * min(step, nsteps - 1);
#pragma unroll
        for (int i = 0; i < XH4; ++i) dst[i] = *reinterpret_cast<const u4_t *>(xb + xoff[i]);
    };

    // Slice S (compile-time) of chunk `chunk`: load to registers / store to LDS.
    auto fetch_slice = [&](int chunk, auto s_c, piece_t (&dst)[NPT]) __attribute__((always_inline)) {
        constexpr int S = decltype(s_c)::value;
        const int cc = min(chunk, nch - 1);
        const uint8_t *src = wbase + (size_t)cc * GROW;
#pragma unroll
        for (int i = 0; i < NPT; ++i) {
            if constexpr (QT == XQ_Q6_K) {
                // every lane issues the same three loads (see the staging note)
                const int sh = ((c_begin + cc) & 1) * 2;
                const uint8_t *row = src + wsrc[S][i];
                const u2a4_t v = *reinterpret_cast<const u2a4_t *>(row - sh + wpo[i]);
                const uint32_t s0 = *reinterpret_cast<const uint16_t *>(row + 206);
                const uint32_t s1 = *reinterpret_cast<const uint16_t *>(row + 208);
                dst[i] = u4_t{v[0], v[1], s0, s1};
            } else {
                dst[i] = *reinterpret_cast<const piece_t *>(src + wsrc[S][i]);
            }
        }
    };
    // into chunk buffer wbuf, which holds local chunks of its parity
    auto store_slice = [&](int wbuf, auto s_c, const piece_t (&src)[NPT]) __attribute__((always_inline)) {
        constexpr int S = decltype(s_c)::value;
        uint8_t *buf = wsm[wbuf];
#pragma unroll
        for (int i = 0; i < NPT; ++i) {
            if constexpr (QT == XQ_Q6_K) {
                // the 27th piece: halfwords 206 and 208 (sh = 2), or 208 then two bytes
                // never read (sh = 0)
                const bool odd = ((c_begin ^ wbuf) & 1) != 0;
                const uint32_t tail = __builtin_amdgcn_perm(src[i][3], src[i][2], odd ? 0x05040100u : 0x05040504u);
                if (wvalid[i])
                    *reinterpret_cast<u2_t *>(buf + S * RS * WROW + wdst[i]) =
                        wlast[i] ? u2_t{tail, 0u} : u2_t{src[i][0], src[i][1]};
            } else {
                if (wvalid[i]) *reinterpret_cast<piece_t *>(buf + S * RS * WROW + wdst[i]) = src[i];
            }
        }
    };

    // ---- prologue. LDS: chunk 0, slices 0 and 1 of chunk 1, X(0), X(1).
    // Registers: X(2) (X(2) .. X(PD+1) for fp16 X), the slices written by steps
    // 0 .. PD-1 (chunk 1 slices 2 .. PD+1), the raw weight words of steps 0 and 1,
    // and the A and decoded B fragments of step 0.
    {
        // All ten slice loads are issued before the first store (one memory round
        // trip, not ten in a row).
        piece_t tmp[10][NPT];
        fetch_slice(0, std::integral_constant<int, 0>{}, tmp[0]);
        fetch_slice(0, std::integral_constant<int, 1>{}, tmp[1]);
        fetch_slice(0, std::integral_constant<int, 2>{}, tmp[2]);
        fetch_slice(0, std::integral_constant<int, 3>{}, tmp[3]);
        fetch_slice(0, std::integral_constant<int, 4>{}, tmp[4]);
        fetch_slice(0, std::integral_constant<int, 5>{}, tmp[5]);
        fetch_slice(0, std::integral_constant<int, 6>{}, tmp[6]);
        fetch_slice(0, std::integral_constant<int, 7>{}, tmp[7]);
        fetch_slice(1, std::integral_constant<int, 0>{}, tmp[8]);
        fetch_slice(1, std::integral_constant<int, 1>{}, tmp[9]);
        store_slice(0, std::integral_constant<int, 0>{}, tmp[0]);
        store_slice(0, std::integral_constant<int, 1>{}, tmp[1]);
        store_slice(0, std::integral_constant<int, 2>{}, tmp[2]);
        store_slice(0, std::integral_constant<int, 3>{}, tmp[3]);
        store_slice(0, std::integral_constant<int, 4>{}, tmp[4]);
        store_slice(0, std::integral_constant<int, 5>{}, tmp[5]);
        store_slice(0, std::integral_constant<int, 6>{}, tmp[6]);
        store_slice(0, std::integral_constant<int, 7>{}, tmp[7]);
        if (nch > 1) {
            store_slice(1, std::integral_constant<int, 0>{}, tmp[8]);
            store_slice(1, std::integral_constant<int, 1>{}, tmp[9]);
        }
        fetch_slice(1, std::integral_constant<int, 2>{}, wr[0]);
        fetch_slice(1, std::integral_constant<int, 3>{}, wr[1]);
        fetch_slice(1, std::integral_constant<int, 4>{}, wr[2]);
        fetch_slice(1, std::integral_constant<int, 5>{}, wr[3]);
        static_assert(PD == 4, "prologue fills a ring of 4");
    }
    if constexpr (XH) {
        fetch_xh(0, xh[0]);
        store_xh(0, xh[0]);
        fetch_xh(1, xh[1]);
        store_xh(1, xh[1]);
#pragma unroll
        for (int j = 0; j < PD; ++j) fetch_xh(2 + j, xh[j]);
    } else {
        fetch_x(0);
        store_x(0);
        fetch_x(1);
        store_x(1);
        fetch_x(2);
    }
    __syncthreads();
    // raw weight words of steps s and s+1 (rwd/rwq[s & 1]), read two steps ahead
    uint32_t rwd[2][JT], rwq[2][JT][NRAW];
    load_a(0, afr[0]);
    read_b(0, std::integral_constant<int, 0>{}, rwd[0], rwq[0]);
    read_b(0, std::integral_constant<int, 1>{}, rwd[1], rwq[1]);
    decode_b(std::integral_constant<int, 0>{}, rwd[0], rwq[0], bfr[0]);
    // Step 0 writes X(2) into xs[0]: every wave's read of X(0) from it must be done
    // first (in the loop the step-end barrier separates a buffer's reads from its
    // next write; here nothing else would).
    __syncthreads();

    for (int ch = 0; ch < nch; ++ch) {
        // Step s = 8 ch + blk. At its start: LDS holds X(s+1) and every slice of
        // the chunks of steps s+1 and s+2; afr/bfr[P] hold the fragments of step s;
        // rwd/rwq[P ^ 1] the raw weight words of step s+1; xr (or xh[s % PD]) holds
        // X(s+2); wr[s % PD] the slice this step writes. Slice u = s + 2 (slice u % 8
        // of chunk u / 8 + 1) is written at step s, so a chunk is complete two
        // steps before its first block is used, and a buffer is rewritten only
        // after the raw reads of its previous chunk are done.
        auto step_body = [&](auto blk_c) __attribute__((always_inline)) {
            constexpr int blk = decltype(blk_c)::value;
            constexpr int P = blk & 1;
            constexpr int RG = blk % PD;                 // ring slot of this step
            constexpr int B1 = (blk + 1) & 7;            // block of step s+1
            constexpr int B2 = (blk + 2) & 7;            // block of step s+2
            const int s = ch * 8 + blk;
            // (1) LDS reads first, so that their latency is spent under the MFMAs:
            // A fragments of step s+1, raw weight words of step s+2.
            load_a(P ^ 1, afr[P ^ 1]);
            read_b((ch + ((blk + 2) >> 3)) & 1, std::integral_constant<int, B2>{}, rwd[P],
                   rwq[P]);
            // (2) staging: X(s+2) -> xs[P] (X(s) was read during step s-1), then
            // fetch the X that step s+PD writes (s+3 for f32 X, one step ahead);
            // slice u = s+2 -> LDS, then fetch the slice step s+PD writes.
            if constexpr (XH) {
                store_xh(P, xh[RG]);        // X(s+2), fetched at step s-PD
                fetch_xh(s + 2 + PD, xh[RG]);
            } else {
                store_x(P);                 // X(s+2), fetched at step s-1
                fetch_x(s + 3);
            }
            {
                const int wc = ch + 1 + ((blk + 2) >> 3);  // chunk receiving the slice
                if (wc < nch) store_slice(wc & 1, std::integral_constant<int, B2>{}, wr[RG]);
                fetch_slice(ch + 1 + ((blk + PD + 2) >> 3),
                            std::integral_constant<int, (blk + PD + 2) & 7>{}, wr[RG]);
            }
            // (3) this step's MFMAs, with the decode of step s+1's weights (raw
            // words read during step s-1) spread between them.
            decode_b(std::integral_constant<int, B1>{}, rwd[P ^ 1], rwq[P ^ 1], bfr[P ^ 1]);
#pragma unroll
            for (int j = 0; j < JT; ++j)
#pragma unroll
                for (int i = 0; i < IT; ++i) {
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(afr[P][i][0], bfr[P][j][0], acc[i][j], 0, 0, 0);
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(afr[P][i][1], bfr[P][j][1], acc[i][j], 0, 0, 0);
                }
            // Instruction order for the scheduler: LDS reads, global loads, LDS
            // writes, then each MFMA followed by a few VALU instructions.
            __builtin_amdgcn_sched_group_barrier(0x100, 32, 0);  // DS reads
            __builtin_amdgcn_sched_group_barrier(0x020, 16, 0);  // VMEM reads
            __builtin_amdgcn_sched_group_barrier(0x200, 16, 0);  // DS writes
#pragma unroll
            for (int q = 0; q < 2 * IT * JT; ++q) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
                __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);  // VALU
            }
            __syncthreads();
        };
        step_body(std::integral_constant<int, 0>{});
        step_body(std::integral_constant<int, 1>{});
        step_body(std::integral_constant<int, 2>{});
        step_body(std::integral_constant<int, 3>{});
        step_body(std::integral_constant<int, 4>{});
        step_body(std::integral_constant<int, 5>{});
        step_body(std::integral_constant<int, 6>{});
        step_body(std::integral_constant<int, 7>{});
    }

    // ---- epilogue. Lane (c, h) holds D[8 (r/4) + 4h + r%4][c], r = 0..15.
    // Indices come from an opaque copy of the thread id so that none of this is
    // computed before the K loop and held in registers across it.
    int etid = threadIdx.x;
    asm volatile("" : "+v"(etid));
    if constexpr (EPI == EPI_SWIGLU) __syncthreads();  // the X buffers become scratch
    const int e_lane = etid & 63, e_wave = etid >> 6;
    const int e_wm = e_wave / WVN, e_wn = e_wave % WVN;
    const int e_c = e_lane & 31, e_h = e_lane >> 5;
#pragma unroll
    for (int i = 0; i < IT; ++i) {
#pragma unroll
        for (int j = 0; j < JT; ++j) {
            const int tile_col = (e_wn * JT + j) * 32;
            const int trow = m0 + e_wm * IT * 32 + i * 32 + 4 * e_h;
            if constexpr (EPI == EPI_SWIGLU) {
                // Columns 0..15 of the tile are gate rows, 16..31 the up rows of the
                // same 16 outputs. The wave writes the tile to its own LDS slot
                // transposed ([column][row], rows padded to 36 floats), then each lane
                // reads four rows of one gate column and of its up column and
                // finishes 2 x 4 outputs. Wave-scope fences order the lanes' exchange
                // (and this tile's writes after the previous tile's reads).
                float *slot = reinterpret_cast<float *>(smem) + e_wave * (32 * 36);
                wave_lds_sync();
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4)
                    *reinterpret_cast<f4_t *>(slot + e_c * 36 + 8 * g4 + 4 * e_h) =
                        f4_t{acc[i][j][4 * g4], acc[i][j][4 * g4 + 1], acc[i][j][4 * g4 + 2],
                             acc[i][j][4 * g4 + 3]};
                wave_lds_sync();
                const int cc = e_lane & 15;
                const int o = tn * (NW / 2) + (tile_col >> 1) + cc;
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    const int q = (e_lane >> 4) + 4 * half;  // row quad 0..7
                    const f4_t g = *reinterpret_cast<const f4_t *>(slot + cc * 36 + 4 * q);
                    const f4_t u = *reinterpret_cast<const f4_t *>(slot + (cc + 16) * 36 + 4 * q);
                    const int t0 = m0 + e_wm * IT * 32 + i * 32 + 4 * q;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (t0 + e < T && o < n) Y[(size_t)(t0 + e) * ldy + o] = silu_fast(g[e]) * u[e];
                }
            } else {
                const int o = tn * NW + tile_col + e_c;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int t = trow + 8 * (r >> 2) + (r & 3);
                    if (t < T && o < n) {
                        float *y = Y + (size_t)t * ldy + o;
                        // A K split stores its partial sums in block `split` of Y
                        // (the workspace, pstride floats apart; a sum kernel adds
                        // them in split order). RESIDUAL without a split: one
                        // writer per element reads R and stores R + acc.
                        if constexpr (SPLIT)
                            y[(size_t)split * pstride] = acc[i][j][r];
                        else if constexpr (EPI == EPI_RESIDUAL)
                            *y = *y + acc[i][j][r];
                        else
                            *y = acc[i][j][r];
                    }
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Cooperative decode: 8 waves (512 threads, two per SIMD) on a tile of MT token
// rows x NW weight rows: 256 x 192 (waves 4 x 2) or 512 x 96 (waves 8 x 1). Either
// way each wave owns 64 x 96 outputs (2 x 3 MFMA tiles of 32 x 32, 96 accumulators).
//  - B: every weight block of the tile is decoded once per workgroup, by all 512
//    threads, into an fp16 tile in LDS kept in B-fragment order, so that a wave
//    reads a B fragment with one 16-byte LDS load per lane (vs decoding in each
//    wave the columns it uses: 4 or 8 times the decode work). The 512 x 96 tile
//    decodes each block once per 512 token rows.
//  - A: X comes from the workspace already in A-fragment order (x_to_frag_kernel),
//    so each wave loads its A fragments straight from global memory, one 16-byte
//    load per lane and fragment, AD steps ahead into a ring of registers. X thus
//    costs no LDS traffic at all (measured: staging X through LDS and reading it
//    back cost as much as the decode).
// LDS: four B buffers of NW x 64 bytes and two raw chunk buffers of NW x 144 (Q4_0)
// or NW x 272 (Q8_0) bytes.
//
// Per step s (one 32-k block), with one barrier at its end:
//   (a) read the second half (k 16..31) of step s's B fragments, and block s+2's
//       raw words from its chunk;
//   (b) the MFMAs of the first half, whose B fragments were read during step s-1,
//       with the staging of slice (s+2) % 8 (NW / 8 whole rows) of a raw weight chunk;
//   (c) the MFMAs of the second half, with the decode of block s+2 into B buffer
//       (s+2) % 4, and the A loads of step s+AD;
//   (d) read the first half of step s+1's B fragments, then the barrier.
// Decoded B lives in a ring of four LDS buffers; raw chunks take two buffers,
// chunk c being filled during steps 8c-10 .. 8c-3 and decoded during steps
// 8c-2 .. 8c+5.
//
// Decode assignment: 256 x 192 tiles give each thread one Q4_0 word whole and one
// nibble half of another, or three Q8_0 words; 512 x 96 tiles give each thread
// one or two units of 4 weights. Within each half wave (32 lanes) the stores cover
// 256 contiguous bytes of one fragment half, so they are free of bank conflicts.
template <int QT, int EPI, bool SPLIT, int MT = 256, int AD = 2>
__global__ __launch_bounds__(512)
void gemm_f16_coop_kernel(const uint8_t *__restrict__ W, const uint16_t *__restrict__ Xf,
                          float *__restrict__ Y, float *__restrict__ Ps, long pstride, int n,
                          int ldy, int k, int T, int tiles_m, int tiles_n, int splits) {
    using CT = ChunkTraits<QT>;
    static_assert(MT == 256 || MT == 512, "tile: 256 x 192 or 512 x 96");
    constexpr bool XQ = coop_xq<QT>();
    static_assert(!XQ || MT == 512 || (QT != XQ_F16 && QT != XQ_Q6_K), "F16, Q6_K: 512 x 96 tiles only");
    constexpr int NW = MT == 256 ? 192 : 96;        // weight rows per tile
    constexpr int WN = NW / 96;                     // waves across the weight rows (2 or 1)
    constexpr int BB = CT::BB;                      // 18 / 34
    constexpr int IT = 2, JT = 3;                   // per wave: 64 rows x 96 weight rows
    constexpr int U4 = CT::U4;                      // 9 / 17
    constexpr int WROW = CT::ROW;                   // 144 / 272
    constexpr int WBUF = NW * WROW;                 // raw chunk buffer
    constexpr int BBUF = NW * 32 * 2;               // B(s): NW/32 tiles x 2 halves x 64 lanes x 16 B
    constexpr int NBB = 4;                          // B buffers
    constexpr int PD = 4;                           // weight staging ring depth (steps)
    // s_waitcnt lgkmcnt(JT): the barrier lets the JT B reads just issued stay in flight
    constexpr int WAITCNT_LGKM_JT = 0xC07F | (JT << 8);
    static_assert(JT <= 15, "lgkmcnt field");
    constexpr int LOOP_BYTES = NBB * BBUF + 2 * WBUF;
    constexpr int EPI_BYTES = 8 * 32 * 36 * 4;
    __shared__ __attribute__((aligned(16))) uint8_t smem[LOOP_BYTES > EPI_BYTES ? LOOP_BYTES : EPI_BYTES];
    uint8_t *const bsm = smem;
    uint8_t *const wsm0 = smem + NBB * BBUF;
    static_assert(WBUF % 16 == 0 && BBUF % 16 == 0, "16-byte aligned carve-up");
    static_assert(8 % PD == 0 && 8 % AD == 0 && 8 % NBB == 0, "rings follow the step within a chunk");

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;

    // Workgroup -> tile, XCD-aware (as in gemm_f16_kernel).
    const int total = tiles_m * tiles_n * splits;
    int logical;
    {
        const int id = blockIdx.x;
        const int per = (total + 7) / 8;
        const int xcd = id & 7, slot = id >> 3;
        const int full = total - 8 * (per - 1);
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
    const int nch = c_end - c_begin;
    if (nch <= 0) return;
    const int nsteps = 8 * nch;
    constexpr int GROW = chunk_grow<QT>();          // a row chunk's bytes in the weight
    const uint32_t row_bytes = XQ ? (uint32_t)(k >> 8) * GROW : (uint32_t)(k >> 5) * BB;

    // A fragments: 32-row tile rt, 16-k slice kk at fragment rt * (k / 16) + kk of
    // the workspace (1 KB each; this lane's 16 bytes at 16 lane). Row tiles past
    // the padded T read the last one; their outputs are never stored.
    const int rt_last = ((T + 31) >> 5) - 1;
    const uint8_t *abase[IT];
#pragma unroll
    for (int i = 0; i < IT; ++i) {
        const int rt = min((m0 >> 5) + wm * IT + i, rt_last);
        abase[i] = reinterpret_cast<const uint8_t *>(Xf) +
                   ((size_t)rt * (k >> 4) + (size_t)c_begin * 16) * 1024 + lane * 16;
    }

    // Weight staging: slice S of a chunk = its rows 24 S .. 24 S + 23, whole (216 /
    // 408 16-byte pieces; thread t < 24 U4 copies piece t % U4 of slice row t / U4).
    // IQ4_XS moves 8-byte pieces (17 per 136-byte row chunk).
    constexpr int RS = NW / 8;
    constexpr int SP = RS * U4;
    constexpr int PIECE = chunk_piece<QT>();
    static_assert(SP <= 512, "one piece per thread");
    static_assert(U4 * PIECE == WROW, "whole pieces per row chunk");
    const bool wvalid = tid < SP;
    const int wff = wvalid ? tid : 0;
    const int wrr = wff / U4, wpp = wff % U4;
    const int wdst = wrr * WROW + PIECE * wpp;
    uint32_t wsrc[8];
#pragma unroll
    for (int S = 0; S < 8; ++S) {
        int gr = f16_weight_row<EPI, NW>(tn, S * RS + wrr, n);
        gr = gr < 0 ? 0 : gr;
        // Q6_K: the row's start; the piece offset is added per chunk
        wsrc[S] = (uint32_t)gr * row_bytes + (QT == XQ_Q6_K ? 0 : PIECE * wpp);
    }
    const uint8_t *wbase = W + (size_t)c_begin * GROW;

    // B fragment (tile jj, half q): 16 bytes of lane `lane` in fragment (wn 3 + jj, q).
    const int boff = (wn * JT * 2 * 64 + lane) * 16;

    // Decode: whole word w0 of row r0, nibble half e1 of word w1 of row r1. Raw
    // offsets inside a chunk buffer (block 0); fragment offsets inside a B buffer:
    // tile r / 32, half, lane (r % 32, w / 2), byte 8 (w % 2).
    //  - whole words: wave v takes rows 16 v .. 16 v + 15; its lane l the word
    //    2 (l / 32) + l % 2 of row 16 v + (l / 2) % 16;
    //  - nibble halves: the 32-lane group g = t / 32 takes nibble half g % 2 of words
    //    2 ((g / 2) % 2) + {0, 1} of rows 128 + 16 (g / 4) .. + 15; lane l of the
    //    group word 2 ((g / 2) % 2) + l % 2 of row 128 + 16 (g / 4) + l / 2.
    // Q8_0 (1536 words of 4 int8 per block): thread t decodes 3 words; 32-lane group
    // g = t / 32 + 16 i (i = 0..2) takes rows 16 (g / 4) .. + 15, fragment half
    // (g / 2) % 2, lane half g % 2: lane l of the group word 4 ((g / 2) % 2) +
    // 2 (g % 2) + l % 2 of row 16 (g / 4) + l / 2.
    // 512 x 96 tiles (768 units of 4 weights per block): unit = one Q8_0 word, or
    // one nibble half of a Q4_0 word. 32-lane group g (g = t / 32, and 16 + t / 32
    // for t < 256) takes rows 16 (g / 4) .. + 15, fragment half (g / 2) % 2 and lane
    // half g % 2; its lane l the word 2 (g % 2) + l % 2 of that lane half (Q4_0,
    // nibble half (g / 2) % 2) or 4 ((g / 2) % 2) + 2 (g % 2) + l % 2 (Q8_0), of row
    // 16 (g / 4) + l / 2.
    constexpr bool UNITS = NW == 96;
    constexpr int NDW = UNITS ? 2 : (QT == Q4_0) ? 2 : 3;  // words read per thread per step
    int sraw[NDW], qraw[NDW], bdst[NDW];
    uint32_t nshift[NDW] = {};
    const bool has2 = !UNITS || tid < 256;          // second unit (UNITS only; wave-uniform)
    if constexpr (UNITS) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int g = i == 0 ? (tid >> 5) : 16 + ((tid >> 5) & 7);
            const int q = (g >> 1) & 1, hh = g & 1;
            const int r = 16 * (g >> 2) + ((tid & 31) >> 1);
            const int w = (QT == Q4_0) ? 2 * hh + (tid & 1) : 4 * q + 2 * hh + (tid & 1);
            sraw[i] = r * WROW;
            qraw[i] = sraw[i] + 4 * w;
            bdst[i] = (((r >> 5) * 2 + q) * 64 + hh * 32 + (r & 31)) * 16 + 8 * (tid & 1);
            nshift[i] = 4 * q;
        }
    } else if constexpr (QT == Q4_0) {
        const int r0 = 16 * (tid >> 6) + ((tid >> 1) & 15), w0 = 2 * ((tid >> 5) & 1) + (tid & 1);
        const int g1 = tid >> 5;
        const int r1 = 128 + 16 * (g1 >> 2) + ((tid & 31) >> 1), w1 = 2 * ((g1 >> 1) & 1) + (tid & 1);
        const int e1 = g1 & 1;
        sraw[0] = r0 * WROW; qraw[0] = sraw[0] + 4 * w0;
        sraw[1] = r1 * WROW; qraw[1] = sraw[1] + 4 * w1;
        bdst[0] = (((r0 >> 5) * 2) * 64 + (w0 >> 1) * 32 + (r0 & 31)) * 16 + 8 * (w0 & 1);
        bdst[1] = (((r1 >> 5) * 2 + e1) * 64 + (w1 >> 1) * 32 + (r1 & 31)) * 16 + 8 * (w1 & 1);
        nshift[1] = 4 * e1;
    } else {
#pragma unroll
        for (int i = 0; i < NDW; ++i) {
            const int g = (tid >> 5) + 16 * i;
            const int q = (g >> 1) & 1, hh = g & 1;
            const int r = 16 * (g >> 2) + ((tid & 31) >> 1), w = 4 * q + 2 * hh + (tid & 1);
            sraw[i] = r * WROW;
            qraw[i] = sraw[i] + 4 * w;
            bdst[i] = (((r >> 5) * 2 + q) * 64 + hh * 32 + (r & 31)) * 16 + 8 * (tid & 1);
        }
    }

    f16v_t acc[IT][JT];
#pragma unroll
    for (int i = 0; i < IT; ++i)
#pragma unroll
        for (int j = 0; j < JT; ++j) acc[i][j] = f16v_t{};

    auto fetch_slice = [&](int chunk, auto s_c, u4_t &dst) __attribute__((always_inline)) {
        constexpr int S = decltype(s_c)::value;
        const uint8_t *src = wbase + (size_t)min(chunk, nch - 1) * GROW + wsrc[S];
        if constexpr (QT == XQ_Q6_K) {
            // src: this row's chunk start, sh bytes past a dword boundary. Every lane
            // issues the same three loads (the 27th piece's lanes use the halfwords,
            // assembled when stored, so that nothing here waits for a load).
            const int sh = ((c_begin + min(chunk, nch - 1)) & 1) * 2;
            const bool last = wpp == U4 - 1;
            const u2a4_t v = *reinterpret_cast<const u2a4_t *>(src - sh + (last ? 200 : PIECE * wpp));
            const uint32_t s0 = *reinterpret_cast<const uint16_t *>(src + 206);
            const uint32_t s1 = *reinterpret_cast<const uint16_t *>(src + 208);
            dst = u4_t{v[0], v[1], s0, s1};
        } else if constexpr (PIECE == 16) {
            dst = *reinterpret_cast<const u4_t *>(src);
        } else {
            const u2_t v = *reinterpret_cast<const u2_t *>(src);
            dst = u4_t{v[0], v[1], 0u, 0u};
        }
    };
    auto store_slice = [&](int wbuf, auto s_c, const u4_t &src) __attribute__((always_inline)) {
        constexpr int S = decltype(s_c)::value;
        uint8_t *dst = wsm0 + wbuf * WBUF + S * RS * WROW + wdst;
        if constexpr (QT == XQ_Q6_K) {
            // the 27th piece: chunk bytes 208 - sh .. 211 - sh (sh = 2: halfwords 206 and
            // 208; sh = 0: halfword 208, then two bytes never read)
            const bool odd = ((c_begin ^ wbuf) & 1) != 0;
            const uint32_t tail = __builtin_amdgcn_perm(src[3], src[2], odd ? 0x05040100u : 0x05040504u);
            if (wvalid) *reinterpret_cast<u2_t *>(dst) = wpp == U4 - 1 ? u2_t{tail, 0u} : u2_t{src[0], src[1]};
        } else if constexpr (PIECE == 16) {
            if (wvalid) *reinterpret_cast<u4_t *>(dst) = src;
        } else {
            if (wvalid) *reinterpret_cast<u2_t *>(dst) = u2_t{src[0], src[1]};
        }
    };

    // Block `blk` (compile-time) of raw chunk buffer `wbuf` -> B buffer `bbuf`, in
    // two parts so that the LDS reads are issued a phase before the math: read_raw
    // fetches this thread's scales and the dwords holding its qs words; decode_store
    // aligns, decodes and stores them.
    // Further types (a unit is weights 4 w .. 4 w + 3 of the step's sub-block or group
    // blk, qraw = sraw + 4 w): Q4_K / Q5_K keep the 16-byte header in hdr, the qs word
    // in lo and (Q5_K) the qh word in hi; F16 the unit's four binary16 values in hv.
    struct RawWords {
        uint32_t d[NDW], lo[NDW], hi[NDW];
        u4_t hdr[XQ ? NDW : 1];
        u2_t hv[XQ ? NDW : 1];
        uint32_t sh;  // Q6_K: the chunk's byte shift in LDS
    };
    auto read_raw = [&](int wbuf, auto blk_c, RawWords &rw) __attribute__((always_inline)) {
        constexpr int blk = decltype(blk_c)::value;
        if constexpr (XQ) {
            const uint8_t *wb = wsm0 + wbuf * WBUF;
#pragma unroll
            for (int i = 0; i < NDW; ++i) {
                if constexpr (QT == XQ_F16) {
                    rw.hv[i] = *reinterpret_cast<const u2_t *>(wb + 2 * qraw[i] - sraw[i] + 64 * blk);
                } else if constexpr (QT == XQ_Q6_K) {
                    // sub-block blk = 4 h + c, unit w: ql bytes 64 h + 32 (c % 2) + 4 w, qh
                    // bytes 128 + 32 h + 4 w (each as the two dwords around them), the
                    // scale byte 192 + 8 h + w / 4 + 2 c, d at 208; chunk byte b sits at
                    // LDS byte sh + b of the row (sh = 2 for odd chunks)
                    constexpr int H = blk >> 2, C = blk & 3;
                    const int sh = ((c_begin ^ wbuf) & 1) * 2;
                    const int w4 = qraw[i] - sraw[i];
                    const uint32_t *ql = reinterpret_cast<const uint32_t *>(wb + sraw[i] + 64 * H + 32 * (C & 1) + w4);
                    const uint32_t *qh = reinterpret_cast<const uint32_t *>(wb + sraw[i] + 128 + 32 * H + w4);
                    rw.lo[i] = ql[0];
                    rw.hi[i] = ql[1];
                    rw.hdr[i][0] = qh[0];
                    rw.hdr[i][1] = qh[1];
                    rw.hdr[i][2] = (uint32_t)(int)*reinterpret_cast<const int8_t *>(
                        wb + sraw[i] + sh + 192 + 8 * H + 2 * C + (w4 >> 4));
                    rw.hdr[i][3] = *reinterpret_cast<const uint16_t *>(wb + sraw[i] + sh + 208);
                    rw.sh = (uint32_t)sh;
                } else if constexpr (QT == XQ_IQ4_XS) {
                    // header (d, scales_h, scales_l); unit w's codes: low nibbles of bytes
                    // 16 blk + 4 w .. (w < 4) or high nibbles of 16 blk + 4 (w - 4) ..
                    const int w4 = qraw[i] - sraw[i];
                    rw.hv[i] = *reinterpret_cast<const u2_t *>(wb + sraw[i]);
                    rw.lo[i] = *reinterpret_cast<const uint32_t *>(wb + sraw[i] + 8 + 16 * blk + (w4 & 15));
                } else {
                    constexpr int QS = QT == XQ_Q5_K ? 48 : 16;  // qs offset in the super-block
                    rw.hdr[i] = *reinterpret_cast<const u4_t *>(wb + sraw[i]);
                    rw.lo[i] = *reinterpret_cast<const uint32_t *>(wb + qraw[i] + QS + 32 * (blk >> 1));
                    if constexpr (QT == XQ_Q5_K) rw.hi[i] = *reinterpret_cast<const uint32_t *>(wb + qraw[i] + 16);
                }
            }
        } else {
            constexpr int SH = (blk * BB + 2) & 3;   // qs start 2 bytes into a dword for even blocks
            const uint8_t *wb = wsm0 + wbuf * WBUF + blk * BB;
#pragma unroll
            for (int i = 0; i < NDW; ++i) {
                rw.d[i] = *reinterpret_cast<const uint16_t *>(wb + sraw[i]);
                if constexpr (SH == 0) {
                    rw.lo[i] = *reinterpret_cast<const uint32_t *>(wb + qraw[i] + 2);
                } else {
                    const uint32_t *al = reinterpret_cast<const uint32_t *>(wb + qraw[i]);
                    rw.lo[i] = al[0];
                    rw.hi[i] = al[1];
                }
            }
        }
    };
    auto decode_store = [&](const RawWords &rw, auto blk_c, auto bbuf_c) __attribute__((always_inline)) {
        constexpr int blk = decltype(blk_c)::value;
        constexpr int SH = XQ ? 0 : (blk * BB + 2) & 3;
        uint8_t *bb = bsm + decltype(bbuf_c)::value * BBUF;
        uint32_t qw[NDW];
#pragma unroll
        for (int i = 0; i < NDW; ++i)
            qw[i] = SH == 0 ? rw.lo[i] : __builtin_amdgcn_alignbyte(rw.hi[i], rw.lo[i], SH);
        // One unit: 4 weights (Q4_0 nibble half `sh` of word w, or Q8_0 word w, or the
        // further types' unit) -> 8 bytes.
        auto unit = [&](int i) __attribute__((always_inline)) {
            if constexpr (QT == XQ_F16) {
                // the binary16 weights themselves (the f32 value rounds back to them)
                *reinterpret_cast<u2_t *>(bb + bdst[i]) = rw.hv[i];
                return;
            }
            uint32_t p[2];
            if constexpr (QT == XQ_Q6_K) {
                // (d sc) (q - 32): d sc is exact, the product rounds once in f32; then
                // binary16 (RNE). q: 4 low bits from ql (high nibble for c >= 2), 2 high
                // bits from qh bits 2 c, 2 c + 1.
                constexpr int C = blk & 3;
                const uint32_t qlw = __builtin_amdgcn_alignbyte(rw.hi[i], rw.lo[i], rw.sh);
                const uint32_t qhw = __builtin_amdgcn_alignbyte(rw.hdr[i][1], rw.hdr[i][0], rw.sh);
                const uint32_t q = ((qlw >> (4 * (C >> 1))) & 0x0F0F0F0Fu) | (((qhw >> (2 * C)) & 0x03030303u) << 4);
                const float ds = fp16_bits_to_f32(rw.hdr[i][3]) * (float)(int)rw.hdr[i][2];
                float w[4];
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    w[c] = ds * (float)((int)((q >> (8 * c)) & 0xFFu) - 32);
                    asm("" : "+v"(w[c]));
                }
                p[0] = h2_bits(h2_t{(_Float16)w[0], (_Float16)w[1]});
                p[1] = h2_bits(h2_t{(_Float16)w[2], (_Float16)w[3]});
            } else if constexpr (QT == XQ_IQ4_XS) {
                // sub-block blk's 6-bit scale ls (nibble of scales_l, 2 bits of scales_h);
                // d (ls - 32) and its product with a grid value are exact in f32
                const uint32_t h0 = rw.hv[i][0], sl = rw.hv[i][1];
                const uint32_t ls = ((sl >> (4 * blk)) & 15u) | (((h0 >> (16 + 2 * blk)) & 3u) << 4);
                const float dl = fp16_bits_to_f32(h0 & 0xFFFFu) * (float)((int)ls - 32);
                const uint32_t g = iq4_grid_bytes((rw.lo[i] >> ((qraw[i] - sraw[i]) >> 2 & 4)) & 0x0F0F0F0Fu);
                float w[4];
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    w[c] = dl * (float)(int8_t)(uint8_t)(g >> (8 * c));
                    asm("" : "+v"(w[c]));
                }
                p[0] = h2_bits(h2_t{(_Float16)w[0], (_Float16)w[1]});
                p[1] = h2_bits(h2_t{(_Float16)w[2], (_Float16)w[3]});
            } else if constexpr (XQ) {
                // Q4_K / Q5_K sub-block blk: (d s) q - dmin m in f32 ((d s) q is exact, so
                // the FMA rounds once, as the subtraction would), then binary16 (RNE).
                uint32_t sc, mn;
                kq_scale_min<blk>(rw.hdr[i], sc, mn);
                const float a = fp16_bits_to_f32(rw.hdr[i][0] & 0xFFFFu) * (float)sc;
                const float b = fp16_bits_to_f32(rw.hdr[i][0] >> 16) * (float)mn;
                uint32_t q = (rw.lo[i] >> (4 * (blk & 1))) & 0x0F0F0F0Fu;
                if constexpr (QT == XQ_Q5_K) q |= ((rw.hi[i] >> blk) & 0x01010101u) << 4;
                float w[4];
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    w[c] = fmaf(a, (float)((q >> (8 * c)) & 0xFFu), -b);
                    // opaque: a fused multiply-add into binary16 would round once, not twice
                    asm("" : "+v"(w[c]));
                }
                p[0] = h2_bits(h2_t{(_Float16)w[0], (_Float16)w[1]});
                p[1] = h2_bits(h2_t{(_Float16)w[2], (_Float16)w[3]});
            } else if constexpr (QT == Q4_0) {
                const h2_t d2 = as_h2(rw.d[i] | (rw.d[i] << 16));
                const h2_t off = {(_Float16)1032.0f, (_Float16)1032.0f};
                const uint32_t nib = (qw[i] >> nshift[i]) & 0x0F0F0F0Fu;
                p[0] = h2_bits((as_h2(magic_pair(nib, SEL_B02)) - off) * d2);
                p[1] = h2_bits((as_h2(magic_pair(nib, SEL_B13)) - off) * d2);
            } else {
                q8_word_to_h4(qw[i], as_h2(rw.d[i] | (rw.d[i] << 16)), p);
            }
            *reinterpret_cast<u2_t *>(bb + bdst[i]) = u2_t{p[0], p[1]};
        };
        if constexpr (UNITS) {
            unit(0);
            if (has2) unit(1);
        } else if constexpr (QT == Q4_0) {
            const h2_t d20 = as_h2(rw.d[0] | (rw.d[0] << 16));
            uint32_t lo02, lo13, hi02, hi13;
            q4_word_decode(qw[0], d20, lo02, lo13, hi02, hi13);
            *reinterpret_cast<u2_t *>(bb + bdst[0]) = u2_t{lo02, lo13};
            *reinterpret_cast<u2_t *>(bb + bdst[0] + 1024) = u2_t{hi02, hi13};
            unit(1);
        } else if constexpr (XQ) {
#pragma unroll
            for (int i = 0; i < NDW; ++i) unit(i);
        } else {
#pragma unroll
            for (int i = 0; i < NDW; ++i) {
                uint32_t p[2];
                q8_word_to_h4(qw[i], as_h2(rw.d[i] | (rw.d[i] << 16)), p);
                *reinterpret_cast<u2_t *>(bb + bdst[i]) = u2_t{p[0], p[1]};
            }
        }
    };
    auto decode_block = [&](int wbuf, auto blk_c, auto bbuf_c) __attribute__((always_inline)) {
        RawWords rw;
        read_raw(wbuf, blk_c, rw);
        decode_store(rw, blk_c, bbuf_c);
    };

    h8_t fa[AD][2][IT];  // A fragments [ring slot][k half][tile]
    h8_t fb[2][JT];      // B fragments [k half][tile]
    auto load_a = [&](int step, h8_t (&dst)[2][IT]) __attribute__((always_inline)) {
        const size_t off = (size_t)min(step, nsteps - 1) * 2048;
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int i = 0; i < IT; ++i)
                dst[q][i] = *reinterpret_cast<const h8_t *>(abase[i] + off + q * 1024);
    };
    auto load_b = [&](auto buf_c, auto q_c) __attribute__((always_inline)) {
        constexpr int q = decltype(q_c)::value;
        const uint8_t *bb = bsm + decltype(buf_c)::value * BBUF + boff + q * 1024;
#pragma unroll
        for (int j = 0; j < JT; ++j) fb[q][j] = *reinterpret_cast<const h8_t *>(bb + j * 2048);
    };
    auto mfma_half = [&](const h8_t (&a)[2][IT], auto q_c) __attribute__((always_inline)) {
        constexpr int q = decltype(q_c)::value;
#pragma unroll
        for (int j = 0; j < JT; ++j)
#pragma unroll
            for (int i = 0; i < IT; ++i)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[q][i], fb[q][j], acc[i][j], 0, 0, 0);
    };

    u4_t wr[PD];      // the slices written by steps s .. s+PD-1

    // ---- prologue (steps -2 and -1): chunk 0 whole and chunk 1 slices 0, 1;
    // blocks 0 and 1 decoded; the first half of step 0's B fragments. The rings hold
    // chunk 1 slices 2 .. PD+1 and the A fragments of steps 0 .. AD-1.
    {
        // All ten slice loads are issued before the first store, so the prologue
        // waits for one memory round trip rather than ten in a row.
        u4_t tmp[10];
        fetch_slice(0, std::integral_constant<int, 0>{}, tmp[0]);
        fetch_slice(0, std::integral_constant<int, 1>{}, tmp[1]);
        fetch_slice(0, std::integral_constant<int, 2>{}, tmp[2]);
        fetch_slice(0, std::integral_constant<int, 3>{}, tmp[3]);
        fetch_slice(0, std::integral_constant<int, 4>{}, tmp[4]);
        fetch_slice(0, std::integral_constant<int, 5>{}, tmp[5]);
        fetch_slice(0, std::integral_constant<int, 6>{}, tmp[6]);
        fetch_slice(0, std::integral_constant<int, 7>{}, tmp[7]);
        fetch_slice(1, std::integral_constant<int, 0>{}, tmp[8]);
        fetch_slice(1, std::integral_constant<int, 1>{}, tmp[9]);
        store_slice(0, std::integral_constant<int, 0>{}, tmp[0]);
        store_slice(0, std::integral_constant<int, 1>{}, tmp[1]);
        store_slice(0, std::integral_constant<int, 2>{}, tmp[2]);
        store_slice(0, std::integral_constant<int, 3>{}, tmp[3]);
        store_slice(0, std::integral_constant<int, 4>{}, tmp[4]);
        store_slice(0, std::integral_constant<int, 5>{}, tmp[5]);
        store_slice(0, std::integral_constant<int, 6>{}, tmp[6]);
        store_slice(0, std::integral_constant<int, 7>{}, tmp[7]);
        if (nch > 1) {
            store_slice(1, std::integral_constant<int, 0>{}, tmp[8]);
            store_slice(1, std::integral_constant<int, 1>{}, tmp[9]);
        }
        // Ring loads in the order the loop issues them (per step: the weight slice,
        // then the A fragments), so that the wait counts the compiler derives at the
        // loop head are the steady-state ones rather than a merge of two orders.
        static_assert(PD == 4 && (AD == 2 || AD == 4), "prologue fills rings of 4 and AD");
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (AD == 2) {
            fetch_slice(1, std::integral_constant<int, 2>{}, wr[0]);
            fetch_slice(1, std::integral_constant<int, 3>{}, wr[1]);
            load_a(0, fa[0]);
            __builtin_amdgcn_sched_barrier(0);
            fetch_slice(1, std::integral_constant<int, 4>{}, wr[2]);
            fetch_slice(1, std::integral_constant<int, 5>{}, wr[3]);
            load_a(1, fa[1]);
        } else {
            fetch_slice(1, std::integral_constant<int, 2>{}, wr[0]);
            load_a(0, fa[0]);
            __builtin_amdgcn_sched_barrier(0);
            fetch_slice(1, std::integral_constant<int, 3>{}, wr[1]);
            load_a(1, fa[1]);
            __builtin_amdgcn_sched_barrier(0);
            fetch_slice(1, std::integral_constant<int, 4>{}, wr[2]);
            load_a(2, fa[2]);
            __builtin_amdgcn_sched_barrier(0);
            fetch_slice(1, std::integral_constant<int, 5>{}, wr[3]);
            load_a(3, fa[3]);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();
    decode_block(0, std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{});
    decode_block(0, std::integral_constant<int, 1>{}, std::integral_constant<int, 1>{});
    __syncthreads();
    load_b(std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{});

    for (int ch = 0; ch < nch; ++ch) {
        auto step_body = [&](auto blk_c) __attribute__((always_inline)) {
            constexpr int blk = decltype(blk_c)::value;
            constexpr int RG = blk % PD;
            constexpr int RA = blk % AD;
            const int s = ch * 8 + blk;
            // Scheduling: the first half's MFMAs each carry an LDS read, a global load
            // or store and a few scalar/vector instructions; the second half's each
            // carry about six decode instructions and a store. Left to itself the
            // scheduler pulls MFMAs up against the reads that feed them and leaves the
            // staging and decode between them. The next step's first-half B reads go
            // last and stay in flight across the barrier: they feed only this wave's
            // registers, and the buffer they read is not rewritten before step s+3.
            RawWords rw;
            load_b(std::integral_constant<int, blk % NBB>{}, std::integral_constant<int, 1>{});
            read_raw((ch + ((blk + 2) >> 3)) & 1, std::integral_constant<int, (blk + 2) & 7>{}, rw);
            mfma_half(fa[RA], std::integral_constant<int, 0>{});
            {
                const int wc = ch + 1 + ((blk + 2) >> 3);  // chunk receiving the slice
                if (wc < nch) store_slice(wc & 1, std::integral_constant<int, (blk + 2) & 7>{}, wr[RG]);
                fetch_slice(ch + 1 + ((blk + PD + 2) >> 3),
                            std::integral_constant<int, (blk + PD + 2) & 7>{}, wr[RG]);
            }
            __builtin_amdgcn_sched_group_barrier(0x100, JT - 1, 0);  // LDS read
            for (int q = 0; q < IT * JT; ++q) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
                __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // global load
                __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // LDS write
                __builtin_amdgcn_sched_group_barrier(0x006, 3, 0);  // VALU / SALU
            }
            __builtin_amdgcn_sched_barrier(0);
            mfma_half(fa[RA], std::integral_constant<int, 1>{});
            decode_store(rw, std::integral_constant<int, (blk + 2) & 7>{},
                         std::integral_constant<int, (blk + 2) % NBB>{});
            load_a(s + AD, fa[RA]);
            for (int q = 0; q < IT * JT; ++q) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);  // MFMA
                __builtin_amdgcn_sched_group_barrier(0x002, 6, 1);  // VALU
                __builtin_amdgcn_sched_group_barrier(0x200, 1, 1);  // LDS write
                __builtin_amdgcn_sched_group_barrier(0x020, 1, 1);  // global load
            }
            __builtin_amdgcn_sched_barrier(0);
            load_b(std::integral_constant<int, (blk + 1) % NBB>{}, std::integral_constant<int, 0>{});
            // Barrier: every earlier LDS operation of this wave (the decode's and the
            // staging's stores) is complete; the JT reads just issued may not be.
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_s_waitcnt(WAITCNT_LGKM_JT);
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        };
        step_body(std::integral_constant<int, 0>{});
        step_body(std::integral_constant<int, 1>{});
        step_body(std::integral_constant<int, 2>{});
        step_body(std::integral_constant<int, 3>{});
        step_body(std::integral_constant<int, 4>{});
        step_body(std::integral_constant<int, 5>{});
        step_body(std::integral_constant<int, 6>{});
        step_body(std::integral_constant<int, 7>{});
    }

    // ---- epilogue (as gemm_f16_kernel, with the (8 / WN) x WN wave layout). The loop's
    // last barrier has retired every LDS access of the K loop.
    int etid = threadIdx.x;
    asm volatile("" : "+v"(etid));
    const int e_lane = etid & 63, e_wave = etid >> 6;
    const int e_wm = e_wave / WN, e_wn = e_wave % WN;
    const int e_c = e_lane & 31, e_h = e_lane >> 5;
#pragma unroll
    for (int i = 0; i < IT; ++i) {
#pragma unroll
        for (int j = 0; j < JT; ++j) {
            const int tile_col = (e_wn * JT + j) * 32;
            const int trow = m0 + e_wm * IT * 32 + i * 32 + 4 * e_h;
            if constexpr (EPI == EPI_SWIGLU) {
                float *slot = reinterpret_cast<float *>(smem) + e_wave * (32 * 36);
                wave_lds_sync();
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4)
                    *reinterpret_cast<f4_t *>(slot + e_c * 36 + 8 * g4 + 4 * e_h) =
                        f4_t{acc[i][j][4 * g4], acc[i][j][4 * g4 + 1], acc[i][j][4 * g4 + 2],
                             acc[i][j][4 * g4 + 3]};
                wave_lds_sync();
                const int cc = e_lane & 15;
                const int o = tn * (NW / 2) + (tile_col >> 1) + cc;
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    const int q = (e_lane >> 4) + 4 * half;
                    const f4_t g = *reinterpret_cast<const f4_t *>(slot + cc * 36 + 4 * q);
                    const f4_t u = *reinterpret_cast<const f4_t *>(slot + (cc + 16) * 36 + 4 * q);
                    const int t0 = m0 + e_wm * IT * 32 + i * 32 + 4 * q;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (t0 + e < T && o < n) Y[(size_t)(t0 + e) * ldy + o] = silu_fast(g[e]) * u[e];
                }
            } else {
                const int o = tn * NW + tile_col + e_c;
                if constexpr (SPLIT) {
                    // This split's partial sums, [T][n] at Ps + split * pstride; the
                    // sum kernel adds the splits (and R) in a fixed order.
                    float *const pb = Ps + (size_t)split * pstride;
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int t = trow + 8 * (r >> 2) + (r & 3);
                        if (t < T && o < n) pb[(size_t)t * n + o] = acc[i][j][r];
                    }
                } else if constexpr (EPI == EPI_RESIDUAL) {
                    // One writer per element: a plain read of R, then R + acc.
                    float rv[16];
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int t = trow + 8 * (r >> 2) + (r & 3);
                        rv[r] = (t < T && o < n) ? Y[(size_t)t * ldy + o] : 0.f;
                    }
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int t = trow + 8 * (r >> 2) + (r & 3);
                        if (t < T && o < n) Y[(size_t)t * ldy + o] = rv[r] + acc[i][j][r];
                    }
                } else {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int t = trow + 8 * (r >> 2) + (r & 3);
                        if (t < T && o < n) Y[(size_t)t * ldy + o] = acc[i][j][r];
                    }
                }
            }
        }
    }
}

// Y = [R +] P_0 + P_1 + ... + P_{splits-1}, element by element in that order: the
// cooperative kernel's split-K partial sums, [T][n] each, pstride floats apart
// (pstride a multiple of 4). DENSE (rows of Y n floats apart): four elements per
// thread, and the thread past the last whole quad takes the 1-3 left over.
// Otherwise one element per thread, Y[t][o] at Y + t ldy + o.
template <int EPI, bool DENSE>
__global__ __launch_bounds__(256) void split_sum_kernel(const float *__restrict__ Ps,
                                                        float *__restrict__ Y, long count,
                                                        long pstride, int splits, int n, int ldy) {
    const long i = (long)blockIdx.x * 256 + threadIdx.x;
    if constexpr (!DENSE) {
        if (i < count) {
            float *y = Y + (size_t)(i / n) * ldy + i % n;
            float a = EPI == EPI_RESIDUAL ? *y : 0.f;
            for (int s = 0; s < splits; ++s) a += Ps[(size_t)s * pstride + i];
            *y = a;
        }
        return;
    }
    const long quads = count >> 2;
    if (i < quads) {
        f4_t a = EPI == EPI_RESIDUAL ? reinterpret_cast<const f4_t *>(Y)[i] : f4_t{0.f, 0.f, 0.f, 0.f};
        auto part = [&](int s) { return reinterpret_cast<const f4_t *>(Ps + (size_t)s * pstride)[i]; };
        // four splits' loads in flight at a time; the additions keep split order
        int s = 0;
        for (; s + 4 <= splits; s += 4) {
            const f4_t p0 = part(s), p1 = part(s + 1), p2 = part(s + 2), p3 = part(s + 3);
            a += p0;
            a += p1;
            a += p2;
            a += p3;
        }
        for (; s < splits; ++s) a += part(s);
        reinterpret_cast<f4_t *>(Y)[i] = a;
    } else if (i == quads) {
        for (long e = 4 * quads; e < count; ++e) {
            float a = EPI == EPI_RESIDUAL ? Y[e] : 0.f;
            for (int s = 0; s < splits; ++s) a += Ps[(size_t)s * pstride + e];
            Y[e] = a;
        }
    }
}

// Y [T][n] (rows ldy apart) = silu(g) * u with g = sum_s G_s[t][o], u = sum_s G_s[t][n + o]
// over the `splits` blocks G_s [T][2n] (pstride floats apart) in order: the gate rows'
// products in columns 0..n-1, the up rows' in n..2n-1.
__global__ void swiglu_apply_kernel(const float *__restrict__ G, float *__restrict__ Y, int T, int n,
                                    int ldy, int splits, long pstride) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= T * n) return;
    const int t = i / n, o = i - t * n;
    const float *g = G + (size_t)t * 2 * n;
    float gs = g[o], us = g[n + o];
    // three splits' loads in flight at a time; the additions keep split order
    int sp = 1;
    for (; sp + 3 <= splits; sp += 3) {
        const float *g0 = g + (size_t)sp * pstride, *g1 = g0 + pstride, *g2 = g1 + pstride;
        const float a0 = g0[o], b0 = g0[n + o], a1 = g1[o], b1 = g1[n + o], a2 = g2[o], b2 = g2[n + o];
        gs += a0;
        us += b0;
        gs += a1;
        us += b1;
        gs += a2;
        us += b2;
    }
    for (; sp < splits; ++sp) {
        gs += g[(size_t)sp * pstride + o];
        us += g[(size_t)sp * pstride + n + o];
    }
    Y[(size_t)t * ldy + o] = silu_fast(gs) * us;
}

namespace {

struct TileChoice {
    int cfg;     // 0: 256x192, 1: 256x128, 2: 128x128, 3: 64x64; waves 1 x 4: 4: 32x128,
                 // 5: 64x128, 6: 128x128
    int splits;
};

constexpr int CFG_MT[4] = {256, 256, 128, 64};
constexpr int CFG_NW[4] = {192, 128, 128, 64};
// Relative MFMA efficiency of each tile shape (bigger wave tiles feed the matrix
// cores with fewer LDS bytes and decode instructions per flop).
constexpr float CFG_EFF[4] = {1.0f, 0.92f, 0.75f, 0.35f};

// allow_split: a K split needs room for its partial sums (a workspace); without
// one the choice is among unsplit tilings only.
TileChoice choose_tiles(const GemmArgs &a, bool allow_split) {
    const bool swiglu = a.epilogue == EPI_SWIGLU;
    const int nchunks = a.k / 256;
    const int cus = 256;
    if (a.T <= SHORT_T || a.qtype == XQ_Q6_K) {
        // One row tile: the matrix-core work is small and the time is the weight
        // stream and its decode. MT x 128 tiles with the waves side by side (no
        // column decoded twice), split along K to fill the resident slots: the
        // split count minimises rounds of workgroups x (chunks per workgroup + one
        // chunk's worth of fixed cost). SwiGLU cannot split: its epilogue is not
        // linear in the partial sums. Q6_K keeps these tiles (several of 128 rows)
        // above 128 rows: its decode is the heaviest, and the cost model's tiles
        // decode each column in two waves (gate/up 2 x 12288 x 4096 at T = 200: 149 us
        // against 203 on 128 x 128; Q4_K there: 108 against 86).
        const int mt = a.T <= 32 ? 32 : a.T <= 64 ? 64 : 128;
        const int cfg = mt == 32 ? 4 : mt == 64 ? 5 : 6;
        const int tn = (a.n + 127) / 128 * ((a.T + mt - 1) / mt);
        if (swiglu || !allow_split) return TileChoice{cfg, 1};
        const long slots = (long)cus * short_tile_waves(a.qtype, mt);
        int best_s = 1;
        long best_c = -1;
        for (int s = 1; s <= nchunks && s <= 32; ++s) {
            const long rounds = ((long)tn * s + slots - 1) / slots;
            const long cost = rounds * ((nchunks + s - 1) / s + 1);
            if (best_c < 0 || cost < best_c) {
                best_c = cost;
                best_s = s;
            }
        }
        return TileChoice{cfg, best_s};
    }
    TileChoice best{3, 1};
    float best_t = 1e30f;
    // The further types' 256 x 192 tile (three B columns per lane, each with its
    // super-block header and code words in flight) spills registers: not taken.
    const bool xq = a.qtype == XQ_Q4_K || a.qtype == XQ_Q5_K || a.qtype == XQ_IQ4_XS;
    for (int cfg = xq ? 1 : 0; cfg < 4; ++cfg) {
        const int MT = CFG_MT[cfg], NW = CFG_NW[cfg];
        const long out_per_tile = swiglu ? NW / 2 : NW;
        const long tm = (a.T + MT - 1) / MT;
        const long tn = (a.n + out_per_tile - 1) / out_per_tile;
        for (int s = 1; s <= 8; ++s) {
            if (s > 1 && (swiglu || !allow_split || s > nchunks)) break;
            const long wgs = tm * tn * s;
            const long rounds = (wgs + cus - 1) / cus;
            // time ~ rounds x work per workgroup / efficiency, plus a split-K cost
            const float work = (float)MT * NW * ((float)a.k / s);
            float t = rounds * work / CFG_EFF[cfg];
            if (s > 1) t *= 1.0f + 0.02f * s;
            if (t < best_t) {
                best_t = t;
                best = TileChoice{cfg, s};
            }
        }
    }
    return best;
}

template <int QT, int EPI, int MT, int NW, bool SPLIT, bool ROW1 = false>
hipError_t launch_cfg(const GemmArgs &a, int splits, const uint16_t *xh, long pstride, hipStream_t s) {
    constexpr int OUT = (EPI == EPI_SWIGLU) ? NW / 2 : NW;
    const int tm = (a.T + MT - 1) / MT;
    const int tn = (a.n + OUT - 1) / OUT;
    const int total = tm * tn * splits;
    if (xh) {
        hipLaunchKernelGGL((gemm_f16_kernel<QT, EPI, MT, NW, SPLIT, true, ROW1>), dim3(total), dim3(256), 0,
                           s, a.W, (const void *)xh, a.Y, a.n, a.ldy, a.k, a.T, tm, tn, splits, pstride);
    } else {
        hipLaunchKernelGGL((gemm_f16_kernel<QT, EPI, MT, NW, SPLIT, false, ROW1>), dim3(total), dim3(256), 0,
                           s, a.W, (const void *)a.X, a.Y, a.n, a.ldy, a.k, a.T, tm, tn, splits, pstride);
    }
    return hipGetLastError();
}

template <int QT, int EPI, bool SPLIT>
hipError_t launch_split(const GemmArgs &a, TileChoice tc, const uint16_t *xh, hipStream_t s,
                        long pstride = 0) {
    {
        switch (tc.cfg) {
        case 0: return launch_cfg<QT, EPI, 256, 192, SPLIT>(a, tc.splits, xh, pstride, s);
        case 1: return launch_cfg<QT, EPI, 256, 128, SPLIT>(a, tc.splits, xh, pstride, s);
        case 2: return launch_cfg<QT, EPI, 128, 128, SPLIT>(a, tc.splits, xh, pstride, s);
        case 3: return launch_cfg<QT, EPI, 64, 64, SPLIT>(a, tc.splits, xh, pstride, s);
        case 4: return launch_cfg<QT, EPI, 32, 128, SPLIT, true>(a, tc.splits, xh, pstride, s);
        case 5: return launch_cfg<QT, EPI, 64, 128, SPLIT, true>(a, tc.splits, xh, pstride, s);
        default: return launch_cfg<QT, EPI, 128, 128, SPLIT, true>(a, tc.splits, xh, pstride, s);
        }
    }
}

// ps: room for the partial sums of a K split (the workspace), or null: then the
// GEMM does not split, and every output has one writer.
template <int QT, int EPI>
hipError_t launch_epi(const GemmArgs &a, const uint16_t *xh, hipStream_t s, float *ps = nullptr) {
    const TileChoice tc = choose_tiles(a, ps != nullptr);
    if constexpr (EPI == EPI_SWIGLU) {
        return launch_split<QT, EPI, false>(a, TileChoice{tc.cfg, 1}, xh, s);
    } else {
        if (tc.splits == 1) return launch_split<QT, EPI, false>(a, tc, xh, s);
        // partial sums into the workspace, then the fixed-order sum (deterministic)
        GemmArgs p = a;
        p.Y = ps;
        p.ldy = a.n;
        const long pstride = part_stride(a.T, a.n);
        hipError_t e = launch_split<QT, EPI, true>(p, tc, xh, s, pstride);
        if (e != hipSuccess) return e;
        const long count = (long)a.T * a.n;
        if (a.ldy == a.n)
            hipLaunchKernelGGL((split_sum_kernel<EPI, true>), dim3((unsigned)((count / 4 + 1 + 255) / 256)),
                               dim3(256), 0, s, ps, a.Y, count, pstride, tc.splits, a.n, a.ldy);
        else
            hipLaunchKernelGGL((split_sum_kernel<EPI, false>), dim3((unsigned)((count + 255) / 256)),
                               dim3(256), 0, s, ps, a.Y, count, pstride, tc.splits, a.n, a.ldy);
        return hipGetLastError();
    }
}

template <int QT>
hipError_t launch_q(const GemmArgs &a, const uint16_t *xh, hipStream_t s, float *ps = nullptr) {
    switch (a.epilogue) {
    case EPI_PLAIN: return launch_epi<QT, EPI_PLAIN>(a, xh, s, ps);
    case EPI_RESIDUAL: return launch_epi<QT, EPI_RESIDUAL>(a, xh, s, ps);
    default: return launch_epi<QT, EPI_SWIGLU>(a, xh, s);
    }
}

// SwiGLU on a short chunk through the workspace: the gate and up rows as one PLAIN
// GEMM over 2n weight rows into G (partial sums of its K split, or the products
// themselves unsplit), then swiglu_apply_kernel.
template <int QT>
hipError_t launch_swiglu_scratch(const GemmArgs &a, const uint16_t *xh, float *G, hipStream_t s) {
    GemmArgs g = a;
    g.epilogue = EPI_PLAIN;
    g.n = 2 * a.n;
    g.Y = G;
    g.ldy = 2 * a.n;
    const TileChoice tc = choose_tiles(g, true);
    const long pstride = part_stride(a.T, 2 * a.n);
    const hipError_t e = tc.splits == 1 ? launch_split<QT, EPI_PLAIN, false>(g, tc, xh, s)
                                        : launch_split<QT, EPI_PLAIN, true>(g, tc, xh, s, pstride);
    if (e != hipSuccess) return e;
    const int count = a.T * a.n;
    hipLaunchKernelGGL(swiglu_apply_kernel, dim3((count + 255) / 256), dim3(256), 0, s, G, a.Y, a.T, a.n, a.ldy,
                       tc.splits, pstride);
    return hipGetLastError();
}

// Most K splits the 4-wave GEMM takes for these sizes: over Q4_0 and Q8_0 (their
// workspace size does not depend on which), or a further type's own choice.
int small_t_splits(int qtype, int T, int n, int k, int epilogue) {
    const bool xq = qtype == XQ_Q4_K || qtype == XQ_Q5_K || qtype == XQ_IQ4_XS || qtype == XQ_Q6_K;
    int m = 1;
    const int types[2] = {xq ? qtype : (int)Q4_0, xq ? qtype : (int)Q8_0};
    for (int q : types) {
        GemmArgs g;
        g.qtype = q;
        g.epilogue = epilogue;
        g.W = nullptr;
        g.X = nullptr;
        g.Y = nullptr;
        g.n = n;
        g.ldy = n;
        g.k = k;
        g.T = T;
        const int sp = choose_tiles(g, true).splits;
        m = sp > m ? sp : m;
    }
    return m;
}

// RMSNorm prologue inside the conversion: x * inv (the row's) * w (the columns')
// in f32, in the order rms_apply_kernel uses, before the rounding to binary16.
__device__ __forceinline__ f4_t rms_scale(f4_t v, float r, const float *__restrict__ w) {
    const f4_t g = *reinterpret_cast<const f4_t *>(w);
    return f4_t{v[0] * r * g[0], v[1] * r * g[1], v[2] * r * g[2], v[3] * r * g[3]};
}

// X [T][k] f32 -> fp16 (RNE) in the k order the GEMM's A fragments take: for
// Q4_0 the order 0, 2, 1, 3 within each group of four, natural for Q8_0. One
// thread writes 8 halves (16 bytes). NORM: the RMSNorm prologue first.
template <int QT, bool NORM>
__global__ __launch_bounds__(256) void x_to_f16_kernel(const float *__restrict__ X,
                                                       uint16_t *__restrict__ Xh, int count8, int k,
                                                       const float *__restrict__ inv,
                                                       const float *__restrict__ nw) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= count8) return;
    f4_t a = reinterpret_cast<const f4_t *>(X)[2 * i];
    f4_t b = reinterpret_cast<const f4_t *>(X)[2 * i + 1];
    if constexpr (NORM) {
        const int row = (int)((long)i * 8 / k), col = i * 8 - row * k;
        a = rms_scale(a, inv[row], nw + col);
        b = rms_scale(b, inv[row], nw + col + 4);
    }
    const u2_t pa = x_pack<QT>(a), pb = x_pack<QT>(b);
    reinterpret_cast<u4_t *>(Xh)[i] = u4_t{pa[0], pa[1], pb[0], pb[1]};
}

// X [T][k] f32 -> fp16 (RNE) in A-fragment order for gemm_f16_coop_kernel: for each
// 32-row tile rt and 16-k slice kk, one 1 KB fragment at index rt * (k / 16) + kk,
// whose lane (c, h) holds row 32 rt + c, k = 16 kk + 8 h .. + 7 in the order of
// x_pack. Rows past T (up to the next multiple of 32) are zero. Thread p converts
// the 16 values of row c = p % 32 in fragment f = p / 32 (64 contiguous bytes) and
// writes lanes (c, 0) and (c, 1): a wave reads 128 contiguous bytes of each of 32
// rows and writes two whole fragments. NORM: the RMSNorm prologue first.
template <int QT, bool NORM>
__global__ __launch_bounds__(256) void x_to_frag_kernel(const float *__restrict__ X,
                                                        uint16_t *__restrict__ Xf, int T, int k,
                                                        int pairs, const float *__restrict__ inv,
                                                        const float *__restrict__ nw) {
    const int p = blockIdx.x * 256 + threadIdx.x;
    if (p >= pairs) return;
    const int c = p & 31;
    const int f = p >> 5;
    const int k16 = k >> 4;
    const int rt = f / k16, kk = f - rt * k16;
    const int row = rt * 32 + c;
    u4_t out0 = u4_t{0u, 0u, 0u, 0u}, out1 = out0;
    if (row < T) {
        const int col = kk * 16;
        const f4_t *src = reinterpret_cast<const f4_t *>(X + (size_t)row * k + col);
        f4_t v[4] = {src[0], src[1], src[2], src[3]};
        if constexpr (NORM) {
#pragma unroll
            for (int j = 0; j < 4; ++j) v[j] = rms_scale(v[j], inv[row], nw + col + 4 * j);
        }
        const u2_t p0 = x_pack<QT>(v[0]), p1 = x_pack<QT>(v[1]);
        const u2_t p2 = x_pack<QT>(v[2]), p3 = x_pack<QT>(v[3]);
        out0 = u4_t{p0[0], p0[1], p1[0], p1[1]};
        out1 = u4_t{p2[0], p2[1], p3[0], p3[1]};
    }
    u4_t *dst = reinterpret_cast<u4_t *>(Xf) + (size_t)f * 64 + c;
    dst[0] = out0;
    dst[32] = out1;
}

}  // namespace

// Partial sums of a K split: block `split` (pstride floats apart) of ps [T][n], each
// stored whole by one workgroup.
long part_stride(int T, int n) { return ((long)T * n + 3) / 4 * 4; }

hipError_t launch_swiglu_apply(const float *G, const GemmArgs &a, int splits, hipStream_t s) {
    const long pstride = part_stride(a.T, 2 * a.n);
    const int count = a.T * a.n;
    hipLaunchKernelGGL(swiglu_apply_kernel, dim3((count + 255) / 256), dim3(256), 0, s, G, a.Y, a.T, a.n, a.ldy,
                       splits, pstride);
    return hipGetLastError();
}

hipError_t launch_split_sum(const GemmArgs &a, const float *ps, int splits, hipStream_t s) {
    const long pstride = part_stride(a.T, a.n);
    const long count = (long)a.T * a.n;
    const bool residual = a.epilogue == EPI_RESIDUAL;
    if (a.ldy == a.n) {
        const dim3 g((unsigned)((count / 4 + 1 + 255) / 256));
        if (residual)
            hipLaunchKernelGGL((split_sum_kernel<EPI_RESIDUAL, true>), g, dim3(256), 0, s, ps, a.Y, count, pstride,
                               splits, a.n, a.ldy);
        else
            hipLaunchKernelGGL((split_sum_kernel<EPI_PLAIN, true>), g, dim3(256), 0, s, ps, a.Y, count, pstride,
                               splits, a.n, a.ldy);
    } else {
        const dim3 g((unsigned)((count + 255) / 256));
        if (residual)
            hipLaunchKernelGGL((split_sum_kernel<EPI_RESIDUAL, false>), g, dim3(256), 0, s, ps, a.Y, count,
                               pstride, splits, a.n, a.ldy);
        else
            hipLaunchKernelGGL((split_sum_kernel<EPI_PLAIN, false>), g, dim3(256), 0, s, ps, a.Y, count, pstride,
                               splits, a.n, a.ldy);
    }
    return hipGetLastError();
}


#ifndef PF_COOP_T512
#define PF_COOP_T512 512
#endif
constexpr int COOP_T512 = PF_COOP_T512;  // smallest T that takes the 512 x 96 tiles

// Split count of the cooperative-decode kernel. PLAIN / RESIDUAL split K when the
// tiles alone would leave CUs idle (any split count; the chunk ranges of the splits
// differ by at most one chunk), but every split keeps at least 4 chunks: a split's
// prologue and the partial-sum traffic cost more than the parallelism buys below
// that. Measured (GEMM kernel, T = 512): Q4_0 4096 x 4096 takes 38.7 us with at
// least 5 chunks per split (3 splits), 34.0 with 4 (4 splits), 45.1 with 8; the
// Q8_0 down projection (k = 12288, 5 splits under any of these) does not change.
// SwiGLU never splits.
static int coop_splits(int MT, int T, int n, int k, int epilogue) {
    if (epilogue == EPI_SWIGLU) return 1;
    const int NW = MT == 256 ? 192 : 96;
    const int tiles = ((T + MT - 1) / MT) * ((n + NW - 1) / NW);
    if (tiles >= 256) return 1;
    int splits = 256 / tiles;
    constexpr int MIN_CHUNKS = 4;
    const int by_k = (k / 256) / MIN_CHUNKS > 1 ? (k / 256) / MIN_CHUNKS : 1;
    if (splits > by_k) splits = by_k;
    if (splits > 16) splits = 16;
    return splits;
}

// The further types this file's GEMMs take on the workspace path: Q4_K, Q5_K and
// IQ4_XS at every T (the 4-wave kernel below 256 rows, the cooperative kernel from
// 256); Q6_K with k % 512 == 0 at every T (the 4-wave kernel up to SHORT_T rows); F16
// above SHORT_T rows. The cooperative kernel takes Q6_K and F16 on its 512-row tile
// only (their 256 x 192 tile's staging would need more than one piece per thread),
// part empty below 512 rows, yet faster there than two or more of the 4-wave kernel's
// row tiles for Q6_K, or F16's own GEMM (gate/up 2 x 12288 x 4096 at T = 300: Q6_K
// 220 -> 104 us, F16 164 -> 93; at T = 200 the 4-wave kernel took 150 us for Q6_K).
bool f16_takes_xq(int qtype, int T, int k) {
    if (qtype == XQ_Q4_K || qtype == XQ_Q5_K || qtype == XQ_IQ4_XS) return true;
    if (qtype == XQ_Q6_K) return k % 512 == 0;
    return qtype == XQ_F16 && T > SHORT_T;
}

// Rows of the cooperative kernel's tile for (qtype, T): 512 from COOP_T512, and for Q6_K
// and F16 (which have no 256-row tile); else 256.
static int coop_mt(int qtype, int T) {
    return (T >= COOP_T512 || qtype == XQ_Q6_K || qtype == XQ_F16) ? 512 : 256;
}

// The further types the f16 GEMM without a workspace (the 4-wave kernel, X rounded in
// each tile, unsplit) takes: Q4_K, Q5_K, IQ4_XS, and Q6_K with k % 512 == 0.
bool f16_direct_takes_xq(int qtype, int k) {
    return qtype == XQ_Q4_K || qtype == XQ_Q5_K || qtype == XQ_IQ4_XS || (qtype == XQ_Q6_K && k % 512 == 0);
}

// Which f16 GEMM runs: the 4-wave kernel (X copied as [T][k]) below 256 rows (Q6_K and
// F16: up to SHORT_T), else the cooperative kernel (X in A-fragment order).
static bool f16_four_wave(int qtype, int T) {
    return (qtype == XQ_Q6_K || qtype == XQ_F16) ? T <= SHORT_T : T < 256;
}

// Byte offset of the partial sums in the workspace, and the floats between splits.
static int64_t ws_x_bytes(int T, int k) { return ((int64_t)(T + 31) / 32 * 32 * k * 2 + 255) / 256 * 256; }
static int64_t ws_pstride(int T, int n) { return part_stride(T, n); }

// Short chunks with the SwiGLU epilogue, on the workspace path: the gate and up rows
// run as one PLAIN GEMM over all 2n weight rows, split along K like the other short
// chunks, into G [T][2n] f32 behind the fp16 X; swiglu_apply_kernel then writes
// Y = silu(gate) * up. Measured faster than the unsplit fused epilogue up to 64 rows
// (gate/up 2 x 12288 x 4096: 28-43 us against 43-46), slower at 100-128 (G's round
// trip grows with T). Without a workspace there is no room for G, and
// the fused epilogue runs unsplit.
constexpr int SWIGLU_SCRATCH_T = 64;
static bool swiglu_via_scratch(int T, int epilogue) { return epilogue == EPI_SWIGLU && T <= SWIGLU_SCRATCH_T; }

int64_t f16_ws_bytes(int qtype, int T, int n, int k, int epilogue) {
    const int64_t xb = (int64_t)(T + 31) / 32 * 32 * k * 2;
    if (swiglu_via_scratch(T, epilogue))
        return ws_x_bytes(T, k) + (int64_t)small_t_splits(qtype, T, 2 * n, k, EPI_PLAIN) * ws_pstride(T, 2 * n) * 4;
    if (f16_four_wave(qtype, T)) {
        const int splits = small_t_splits(qtype, T, n, k, epilogue);
        return splits > 1 ? ws_x_bytes(T, k) + (int64_t)splits * ws_pstride(T, n) * 4 : xb;
    }
    const int splits = coop_splits(coop_mt(qtype, T), T, n, k, epilogue);
    return splits > 1 ? ws_x_bytes(T, k) + (int64_t)splits * ws_pstride(T, n) * 4 : xb;
}

// The cooperative-decode kernel: 256 x 192 tiles, or 512 x 96 (each weight block
// decoded once per 512 token rows instead of per 256: half the decode and weight
// staging per output, at twice the X reads from L2). A K split writes partial sums
// into the workspace behind the fp16 X copy, and split_sum_kernel adds them.
template <int QT, int EPI, int MT>
hipError_t launch_coop(const GemmArgs &a, uint16_t *xh, hipStream_t s) {
    constexpr int NW = MT == 256 ? 192 : 96;
    const int tm = (a.T + MT - 1) / MT;
    const int out_per_tile = EPI == EPI_SWIGLU ? NW / 2 : NW;
    const int tn = (a.n + out_per_tile - 1) / out_per_tile;
    const int splits = coop_splits(MT, a.T, a.n, a.k, EPI);
    const int total = tm * tn * splits;
    if (splits > 1) {
        if constexpr (EPI != EPI_SWIGLU) {
            float *ps = reinterpret_cast<float *>(reinterpret_cast<uint8_t *>(xh) + ws_x_bytes(a.T, a.k));
            const long pstride = (long)ws_pstride(a.T, a.n);
            hipLaunchKernelGGL((gemm_f16_coop_kernel<QT, EPI, true, MT>), dim3(total), dim3(512), 0, s,
                               a.W, xh, a.Y, ps, pstride, a.n, a.ldy, a.k, a.T, tm, tn, splits);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
            const long count = (long)a.T * a.n;
            if (a.ldy == a.n) {
                const long threads = count / 4 + 1;
                hipLaunchKernelGGL((split_sum_kernel<EPI, true>), dim3((unsigned)((threads + 255) / 256)),
                                   dim3(256), 0, s, ps, a.Y, count, pstride, splits, a.n, a.ldy);
            } else {
                hipLaunchKernelGGL((split_sum_kernel<EPI, false>), dim3((unsigned)((count + 255) / 256)),
                                   dim3(256), 0, s, ps, a.Y, count, pstride, splits, a.n, a.ldy);
            }
        }
    } else {
        hipLaunchKernelGGL((gemm_f16_coop_kernel<QT, EPI, false, MT>), dim3(total), dim3(512), 0, s, a.W,
                           xh, a.Y, nullptr, 0L, a.n, a.ldy, a.k, a.T, tm, tn, splits);
    }
    return hipGetLastError();
}

template <int QT, int MT>
hipError_t launch_coop_e(const GemmArgs &a, uint16_t *xh, hipStream_t s) {
    switch (a.epilogue) {
    case EPI_PLAIN: return launch_coop<QT, EPI_PLAIN, MT>(a, xh, s);
    case EPI_RESIDUAL: return launch_coop<QT, EPI_RESIDUAL, MT>(a, xh, s);
    default: return launch_coop<QT, EPI_SWIGLU, MT>(a, xh, s);
    }
}

template <int QT>
hipError_t launch_coop_q(const GemmArgs &a, uint16_t *xh, hipStream_t s) {
    return a.T >= COOP_T512 ? launch_coop_e<QT, 512>(a, xh, s) : launch_coop_e<QT, 256>(a, xh, s);
}

// X -> binary16 into the workspace, in the layout the GEMM for (qtype, T) reads: A-fragment
// order for the cooperative kernel, [T][k] for the 4-wave kernel (f16_four_wave).
hipError_t launch_prepare_x_f16(const GemmArgs &a, void *workspace, hipStream_t s) {
    uint16_t *xh = static_cast<uint16_t *>(workspace);
    if (!f16_four_wave(a.qtype, a.T)) {
        const int count = (a.T + 31) / 32 * 32 * (a.k / 16);  // (row, 16-k slice) pairs
        const dim3 g((count + 255) / 256);
        if (a.norm_inv) {
            if (a.qtype == Q4_0)
                hipLaunchKernelGGL((x_to_frag_kernel<Q4_0, true>), g, dim3(256), 0, s, a.X, xh, a.T, a.k,
                                   count, a.norm_inv, a.norm_w);
            else
                hipLaunchKernelGGL((x_to_frag_kernel<Q8_0, true>), g, dim3(256), 0, s, a.X, xh, a.T, a.k,
                                   count, a.norm_inv, a.norm_w);
        } else if (a.qtype == Q4_0) {
            hipLaunchKernelGGL((x_to_frag_kernel<Q4_0, false>), g, dim3(256), 0, s, a.X, xh, a.T, a.k,
                               count, nullptr, nullptr);
        } else {
            hipLaunchKernelGGL((x_to_frag_kernel<Q8_0, false>), g, dim3(256), 0, s, a.X, xh, a.T, a.k,
                               count, nullptr, nullptr);
        }
        return hipGetLastError();
    }
    const int count8 = a.T * (a.k / 8);
    const dim3 g((count8 + 255) / 256);
    if (a.norm_inv) {
        if (a.qtype == Q4_0)
            hipLaunchKernelGGL((x_to_f16_kernel<Q4_0, true>), g, dim3(256), 0, s, a.X, xh, count8, a.k,
                               a.norm_inv, a.norm_w);
        else
            hipLaunchKernelGGL((x_to_f16_kernel<Q8_0, true>), g, dim3(256), 0, s, a.X, xh, count8, a.k,
                               a.norm_inv, a.norm_w);
    } else if (a.qtype == Q4_0) {
        hipLaunchKernelGGL((x_to_f16_kernel<Q4_0, false>), g, dim3(256), 0, s, a.X, xh, count8, a.k,
                           nullptr, nullptr);
    } else {
        hipLaunchKernelGGL((x_to_f16_kernel<Q8_0, false>), g, dim3(256), 0, s, a.X, xh, count8, a.k,
                           nullptr, nullptr);
    }
    return hipGetLastError();
}

// The f16 GEMM on X already in the workspace (launch_prepare_x_f16 with the same
// qtype, k and T); any split-K partial sums (or the SwiGLU scratch G) go behind it.
hipError_t launch_gemm_f16_prepared(const GemmArgs &a, void *workspace, hipStream_t s) {
    uint16_t *xh = static_cast<uint16_t *>(workspace);
    if (!f16_four_wave(a.qtype, a.T)) {
        switch (a.qtype) {
        case Q4_0: return launch_coop_q<Q4_0>(a, xh, s);
        case Q8_0: return launch_coop_q<Q8_0>(a, xh, s);
        // further types (f16_takes_xq)
        case XQ_Q4_K: return launch_coop_q<XQ_Q4_K>(a, xh, s);
        case XQ_Q5_K: return launch_coop_q<XQ_Q5_K>(a, xh, s);
        case XQ_IQ4_XS: return launch_coop_q<XQ_IQ4_XS>(a, xh, s);
        case XQ_F16: return launch_coop_e<XQ_F16, 512>(a, xh, s);
        case XQ_Q6_K: return launch_coop_e<XQ_Q6_K, 512>(a, xh, s);
        default: return hipErrorInvalidValue;
        }
    }
    // split-K partial sums (or the SwiGLU scratch G) go behind the fp16 X
    float *ps = reinterpret_cast<float *>(reinterpret_cast<uint8_t *>(workspace) + ws_x_bytes(a.T, a.k));
    const bool g = swiglu_via_scratch(a.T, a.epilogue);
    switch (a.qtype) {
    case Q4_0: return g ? launch_swiglu_scratch<Q4_0>(a, xh, ps, s) : launch_q<Q4_0>(a, xh, s, ps);
    case Q8_0: return g ? launch_swiglu_scratch<Q8_0>(a, xh, ps, s) : launch_q<Q8_0>(a, xh, s, ps);
    // further types on the 4-wave kernel (f16_takes_xq)
    case XQ_Q4_K: return g ? launch_swiglu_scratch<XQ_Q4_K>(a, xh, ps, s) : launch_q<XQ_Q4_K>(a, xh, s, ps);
    case XQ_Q5_K: return g ? launch_swiglu_scratch<XQ_Q5_K>(a, xh, ps, s) : launch_q<XQ_Q5_K>(a, xh, s, ps);
    case XQ_IQ4_XS: return g ? launch_swiglu_scratch<XQ_IQ4_XS>(a, xh, ps, s) : launch_q<XQ_IQ4_XS>(a, xh, s, ps);
    case XQ_Q6_K: return g ? launch_swiglu_scratch<XQ_Q6_K>(a, xh, ps, s) : launch_q<XQ_Q6_K>(a, xh, s, ps);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_gemm_f16_ws(const GemmArgs &a, void *workspace, hipStream_t s) {
    const hipError_t e = launch_prepare_x_f16(a, workspace, s);
    if (e != hipSuccess) return e;
    return launch_gemm_f16_prepared(a, workspace, s);
}

hipError_t launch_gemm_f16(const GemmArgs &a, hipStream_t s) {
    switch (a.qtype) {
    case Q4_0: return launch_q<Q4_0>(a, nullptr, s);
    case Q8_0: return launch_q<Q8_0>(a, nullptr, s);
    // further types (f16_direct_takes_xq)
    case XQ_Q4_K: return launch_q<XQ_Q4_K>(a, nullptr, s);
    case XQ_Q5_K: return launch_q<XQ_Q5_K>(a, nullptr, s);
    case XQ_IQ4_XS: return launch_q<XQ_IQ4_XS>(a, nullptr, s);
    case XQ_Q6_K: return launch_q<XQ_Q6_K>(a, nullptr, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace pf
