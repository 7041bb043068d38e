// bf16 attention forward, prefill shape (any T_q), for gfx950.
//
// Method: FlashAttention-style tiling with online softmax (AIInfraGuide
// "3.3 Self-Attention机制深入理解", sections 7.3, 12.2, 12.3): each
// workgroup owns a block of query rows of one (batch, q head), walks the
// key/value tiles of its kv head, keeps a running row maximum m, a running
// exponential sum l and an unnormalised output accumulator in registers,
// rescales them when m grows, and divides by l once at the end.  Scores and
// weights never leave the chip.
//
// gfx950 mapping:
//   * Each wave owns RB blocks of 32 query rows.  It computes S^T = K * Q^T
//     for 32 keys at a time with v_mfma_f32_32x32x16_bf16: one query row per
//     lane column and 16 keys per lane, so a row's maximum and sum are
//     in-lane plus one exchange with lane^32.  Every K fragment read from LDS feeds RB
//     MFMAs, and so does every V fragment: LDS read traffic per FLOP falls
//     as 1/RB.  (At RB = 1 one 32x32x16 MFMA per SIMD per 32 clocks
//     consumes 128 B/clock per CU of LDS reads; LDS was measured to deliver
//     about 139 B/clock per CU to 8 waves.)
//   * The score accumulator layout is the B operand of O^T = V^T * P^T:
//     weights are rounded to bf16 in place and never move between lanes.
//     The V^T A operand comes straight from the row-major V tile with the
//     transposing LDS read ds_read_b64_tr_b16.
//   * K and V tiles go from HBM to LDS with 16-byte buffer loads that write
//     LDS directly (no register staging).  Each 1 KiB load covers whole rows;
//     an XOR swizzle of the 16-byte chunks (chosen through the per-lane
//     source address) keeps the K reads and the transposing V reads free of
//     bank conflicts on the 64-bank LDS.  The tile's first row goes into a
//     per-tile buffer resource, so the lane offsets are constants.
//   * Each step handles one key tile: scores, weights, O += P V.  The two
//     waves on each SIMD overlap one another's matrix-core and vector work;
//     computing the next tile's scores inside the current step (a software
//     pipeline within the wave) measured slower and needs twice the score
//     registers.  LDS holds two K and two V tiles (tile t being read, t+1
//     loading); the loop is unrolled by two so both slots are compile-time
//     offsets.
//   * The K fragments of the score phase are read four MFMA groups ahead of
//     their use, the V^T fragments one key step ahead, both as inline
//     assembly with waits bound to the fragment registers (see score_tile,
//     pv_tile): the compiler otherwise keeps too few reads in flight and
//     stalls the V^T reads behind the tile prefetches.  The P V MFMAs issue
//     at raised wave priority.
//   * Softmax in the exp2 domain: one FMA forms score * scale * log2(e) -
//     base per weight.  No row maximum is taken while the weights stay
//     small: the row sums (which are needed anyway) show when a base must
//     move, and only then is the exact row maximum taken and the weights
//     recomputed (so weights stay below 2^16 and the O rescale is rare; the
//     final O / l is the same for any base).  Row sums add the bf16-rounded
//     weights with v_dot2_f32_bf16, so O stays a convex combination of V's
//     rows.
//   * Causal: key tiles wholly above the diagonal are never visited (per
//     workgroup) or skipped (per wave and row block); only tiles that cross
//     the diagonal or the end of the keys pay for the element mask (Ch. 11
//     "Attention" page, section 11.8.3), using exact tile bounds.
//   * Workgroups run heaviest query tile first (causal work grows along the
//     sequence) and, when the kv-head count allows, all workgroups of one
//     (batch, kv head) run on one XCD so its K/V stay in that XCD's L2; the
//     units are dealt to the XCDs in turn so unequal sequences of a packed
//     batch spread evenly.
//
// Configurations (RB = 1, two waves per SIMD at D = 128): 8 waves x 32 rows
// per workgroup and 128-key tiles for long sequences (one K/V tile in LDS
// serves 256 query rows, one workgroup per CU); 8 waves in two key groups of
// 4 over 128 rows with 64-key tiles for problems whose 128-row workgroups all
// fit on the GPU at once (the key split halves the longest chain of steps);
// 4 waves x 32 rows and 64-key tiles otherwise (two workgroups per CU).
// RB = 2 halves the LDS read traffic per
// FLOP but needs more than 256 registers per lane, i.e. one wave per SIMD,
// and was measured slower: a single wave cannot overlap its own softmax with
// its MFMAs the way two waves of a SIMD overlap each other's.
#include "launch.h"

namespace attn {
namespace {

struct TileCoord {
    int qt, b, hq, hk;
};

// Workgroup id -> (query tile, batch, q head, kv head).
__device__ inline TileCoord map_tile(int id, int B, int H_q, int H_kv, int n_qt, bool causal) {
    const int G = H_q / H_kv;
    const int units = B * H_kv;  // (batch, kv head) pairs
    int qt_rev, unit, g;
    if ((units & 7) == 0) {
        // Dispatch sends workgroup id to XCD (id mod 8).  Every workgroup of
        // one (batch, kv head) unit goes to the XCD unit mod 8, so the unit's
        // K/V is read through one L2; units are dealt to the XCDs in turn, so
        // each XCD holds the same kv head of every sequence (in a packed batch
        // of unequal lengths, contiguous blocks of units left one XCD with
        // over twice the mean work).  Within an XCD, heaviest query tile first.
        const int xcd = id & 7;
        const int slot = id >> 3;
        const int upx = units >> 3;
        const int per = upx * G;
        qt_rev = slot / per;
        const int rem = slot - qt_rev * per;
        const int u = rem / G;
        unit = u * 8 + xcd;
        g = rem - u * G;
    } else {
        const int per = units * G;
        qt_rev = id / per;
        const int rem = id - qt_rev * per;
        unit = rem / G;
        g = rem - unit * G;
    }
    TileCoord t;
    t.qt = causal ? n_qt - 1 - qt_rev : qt_rev;
    t.b = unit / H_kv;
    t.hk = unit - t.b * H_kv;
    t.hq = t.hk * G + g;
    return t;
}

// Scores of one key tile for all RB row blocks of this wave.
template <int BN, int RB>
struct STile {
    f32x16 acc[RB][BN / 32];
};

// S^T = K Q^T for one tile: RB * BN/32 independent MFMA chains over the D/16
// feature steps; each K fragment (one ds_read_b128) feeds RB MFMAs.  The
// fragments are read KP MFMA groups ahead of their use through a ring of
// KP + 1 registers (a slot is refilled one group after its last reader), so
// every read has KP groups of matrix-core time to land.
//
// Fragment (s, kb) of lane (l32, hi) is 16-byte chunk (2s + hi) ^ swz(key)
// of key kb * 32 + l32.  swz depends on the key's low 4 bits only, and 2s
// and hi occupy disjoint bits, so the chunk is (hi ^ swz(l32)) ^ 2s: the
// lane's address for step s is a0 ^ 32s (a0 = its step-0 address; rows
// start at multiples of the row size D * 2 and the xor only changes bits
// below it), and key block kb adds the immediate kb * 32 rows.  Four groups
// ahead measured best (two: -1%, six or eight: no better).
constexpr int kScoreReadAhead = 4;
// Largest share of a row's weight sum one lane may hold before the row's
// exponent base is moved (see the step below).
constexpr float kSumGuard = 65536.f;
template <int D, int BN, int RB, int KOFF, int I>
__device__ __attribute__((always_inline)) inline bf16x8 score_read(uint32_t a0) {
    constexpr int NKB = BN / 32;
    return ds_read_b128_asm<KOFF + (I % NKB) * 32 * D * 2>(a0 ^ (uint32_t)(32 * (I / NKB)));
}
template <int D, int BN, int RB, int KOFF, int KP, int I>
__device__ __attribute__((always_inline)) inline void score_group(STile<BN, RB>& st, bf16x8 (&f)[KP + 1],
                                                                  uint32_t a0,
                                                                  const bf16x8 (&qf)[RB][D / 16]) {
    constexpr int NKB = BN / 32;
    constexpr int NM = NKB * (D / 16);
    if constexpr (I + KP < NM) f[(I + KP) % (KP + 1)] = score_read<D, BN, RB, KOFF, I + KP>(a0);
    constexpr int AFTER = (NM - 1 - I) < KP ? (NM - 1 - I) : KP;  // reads issued after read I
    lds_wait_bind1<AFTER>(f[I % (KP + 1)]);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
        st.acc[rb][I % NKB] =
            __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[I % (KP + 1)], qf[rb][I / NKB], st.acc[rb][I % NKB], 0, 0, 0);
}
template <int D, int BN, int RB, int KOFF, int KP, int... I>
__device__ __attribute__((always_inline)) inline void score_groups(STile<BN, RB>& st, bf16x8 (&f)[KP + 1],
                                                                   uint32_t a0,
                                                                   const bf16x8 (&qf)[RB][D / 16],
                                                                   std::integer_sequence<int, I...>) {
    (score_group<D, BN, RB, KOFF, KP, I>(st, f, a0, qf), ...);
}
template <int D, int BN, int RB, int KOFF, int KP, int... P>
__device__ __attribute__((always_inline)) inline void score_prologue(bf16x8 (&f)[KP + 1], uint32_t a0,
                                                                     std::integer_sequence<int, P...>) {
    ((f[P] = score_read<D, BN, RB, KOFF, P>(a0)), ...);
}
// a0: lane's step-0 address in K slot 0; KOFF: byte offset of the slot.
template <int D, int BN, int RB, int KOFF>
__device__ __attribute__((always_inline)) inline void score_tile(STile<BN, RB>& st, uint32_t a0,
                                                                 const bf16x8 (&qf)[RB][D / 16]) {
    constexpr int NM = (BN / 32) * (D / 16);
    constexpr int KP = kScoreReadAhead < NM - 1 ? kScoreReadAhead : NM - 1;
    static_assert(KP >= 1 && KP < NM && KP <= 15, "prefetch depth");
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
        for (int kb = 0; kb < BN / 32; ++kb) st.acc[rb][kb] = f32x16{};
    }
    bf16x8 f[KP + 1];
    score_prologue<D, BN, RB, KOFF, KP>(f, a0, std::make_integer_sequence<int, KP>{});
    score_groups<D, BN, RB, KOFF, KP>(st, f, a0, qf, std::make_integer_sequence<int, NM>{});
}

// KSPLIT = 2 (short problems whose grid does not fill the GPU): the
// workgroup's waves form two key groups over the same query rows; group g
// walks the g-th half of the workgroup's key tiles with its own K/V ring, so
// the longest chain of steps is halved, and at the end the second group's
// (base, sum, unnormalised O) is merged into the first's through LDS with the
// block-merge rule of AIInfraGuide section 12.3.
template <int D, bool CAUSAL, bool VARLEN, int RB, int BN, int WAVES, int WPE, int KSPLIT = 1>
__global__ __launch_bounds__(64 * WAVES) __attribute__((amdgpu_waves_per_eu(WPE, WPE))) void
prefill_bf16_kernel(const bf16* __restrict__ Q, const bf16* __restrict__ K,
                    const bf16* __restrict__ V, bf16* __restrict__ O, int B, int H_q, int H_kv,
                    int T_q, int T_kv, int n_qt, float c, int neg_q, int window,
                    const int* __restrict__ cu_q, const int* __restrict__ cu_k) {
    static_assert(KSPLIT == 1 || (KSPLIT == 2 && RB == 1), "key split: RB = 1");
    constexpr int RW = WAVES / KSPLIT;            // waves per key group (row waves)
    constexpr int WROWS = 32 * RB;                // query rows per wave
    constexpr int BM = WROWS * RW;                // query rows per workgroup
    constexpr int CPR = D / 8;                    // 16-byte chunks per row
    constexpr int ROWB = D * 2;                   // bytes per row
    constexpr int TILE = BN * ROWB;               // bytes of one K or V tile
    constexpr int NLD = TILE / (1024 * RW);       // 1 KiB loads per wave per tile
    static_assert(NLD * 1024 * RW == TILE, "tile must split into 1 KiB wave loads");

    __shared__ __attribute__((aligned(1024))) unsigned char smem[KSPLIT * 4 * TILE];

    const int tid = threadIdx.x;
    const int wave_id = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches
    const int kg = KSPLIT > 1 ? wave_id / RW : 0;  // key group
    const int wave = wave_id - kg * RW;            // row wave within the group
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int hi = lane >> 5;
    unsigned char* const kring = smem + kg * 4 * TILE;  // 2 K tiles of this key group
    unsigned char* const vring = kring + 2 * TILE;      // 2 V tiles

    const TileCoord tc = map_tile(blockIdx.x, B, H_q, H_kv, n_qt, CAUSAL);

    // Rows of this (sequence, head): contiguous [B][H][T][D] (row stride D),
    // or packed token-major [total][H][D] with the sequence's rows starting at
    // cu[b] (row stride H * D).
    const int SQ = VARLEN ? H_q * D : D;   // row strides in elements
    const int SK = VARLEN ? H_kv * D : D;
    size_t q_base, kv_base;
    if constexpr (VARLEN) {
        const int qs = cu_q[tc.b], ks = cu_k[tc.b];
        T_q = max(cu_q[tc.b + 1] - qs, 0);
        T_kv = max(cu_k[tc.b + 1] - ks, 0);
        q_base = (size_t)qs * SQ + (size_t)tc.hq * D;
        kv_base = (size_t)ks * SK + (size_t)tc.hk * D;
    } else {
        q_base = (size_t)(tc.b * H_q + tc.hq) * T_q * D;
        kv_base = (size_t)(tc.b * H_kv + tc.hk) * T_kv * D;
    }
    const int q0 = tc.qt * BM;
    if (q0 >= T_q) return;  // a short sequence of a packed batch: no rows here
    const uint32_t q_bytes = (uint32_t)((T_q - 1) * SQ + D) * 2;
    const uint32_t kv_bytes = T_kv > 0 ? (uint32_t)((T_kv - 1) * SK + D) * 2 : 0u;
    const auto rQ = make_rsrc(Q + q_base, q_bytes);
    const auto rO = make_rsrc(O + q_base, q_bytes);

    const int off = T_kv - T_q;  // bottom-right causal alignment
    const int row0 = q0 + wave * WROWS;  // first row of this wave
    // Sliding window (causal only): row i sees keys i + off - window + 1 ..
    // i + off.
    const bool windowed = CAUSAL && window > 0;
    auto first_key = [&](int row) { return windowed ? max(0, row + off - window + 1) : 0; };

    // Key ranges: the workgroup's, this wave's, each row block's.
    const int last_row = min(T_q, q0 + BM) - 1;
    const int kv_end = CAUSAL ? max(0, min(T_kv, last_row + off + 1)) : T_kv;
    const int n_kt_wg = (kv_end + BN - 1) / BN;
    const int t_lo_wg = min(first_key(q0) / BN, n_kt_wg);  // tiles left of every row's window are never visited
    // This key group's tiles: [t_lo, n_kt), n_steps steps (the second group's
    // last step may have no tile: n_kt - t_lo < n_steps).
    const int n_steps = (n_kt_wg - t_lo_wg + KSPLIT - 1) / KSPLIT;
    const int t_lo = t_lo_wg + kg * n_steps;
    const int n_kt = min(n_kt_wg, t_lo + n_steps);
    int rb_kv_end[RB], rb_kv_begin[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const int r0 = row0 + rb * 32;
        const int rlast = min(T_q - 1, r0 + 31);
        rb_kv_end[rb] = (r0 >= T_q) ? 0 : (CAUSAL ? max(0, min(T_kv, rlast + off + 1)) : T_kv);
        rb_kv_begin[rb] = first_key(r0);
    }
    const int wave_kv_end = rb_kv_end[RB - 1];  // the last row block sees the most keys
    const int wave_kv_begin = rb_kv_begin[0];   // the first row block starts leftmost
    auto wave_live = [&](int j0) { return j0 < wave_kv_end && j0 + BN > wave_kv_begin; };

    // Q fragments: B operands of S^T = K Q^T (column = query row, 8 features).
    // Rows past T_q read as zero.  A negative scale is folded into Q's sign
    // (exact in bf16), so c > 0 below.  Issued before the tile loads.
    bf16x8 qf[RB][D / 16];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
        for (int s = 0; s < D / 16; ++s) {
            u32x4 w = buf_load_b128(rQ, (uint32_t)((row0 + rb * 32 + l32) * SQ + 16 * s + 8 * hi) * 2);
            if (neg_q) w ^= 0x80008000u;
            qf[rb][s] = __builtin_bit_cast(bf16x8, w);
        }
    }

    // Direct-to-LDS loads of one K or V tile.  Keys past T_kv are outside
    // the buffer range and load as zero.  Tile t uses ring slot (t - t_lo) & 1.
    // The tile's first row is folded into a per-tile buffer resource (base
    // moved to it, range shortened by as much, scalar arithmetic), so each
    // lane's offset within the tile is a constant and the loads need no
    // vector address arithmetic; the range check still zeroes keys past T_kv.
    uint32_t loff[NLD];
#pragma unroll
    for (int n = 0; n < NLD; ++n) {
        const int blk = wave * NLD + n;
        const int p = blk * 64 + lane;  // chunk slot in the tile
        const int row = p / CPR;
        const int logical = (p % CPR) ^ swz<CPR>(row);
        loff[n] = (uint32_t)row * SK * 2 + logical * 16;
    }
    auto issue = [&](const bf16* base, unsigned char* dst, int t) {
        const uint32_t off = (uint32_t)__builtin_amdgcn_readfirstlane(t * BN) * (uint32_t)(SK * 2);
        const auto r = make_rsrc(reinterpret_cast<const unsigned char*>(base) + off, kv_bytes - off);
#pragma unroll
        for (int n = 0; n < NLD; ++n) buf_load_lds16(r, dst + (wave * NLD + n) * 1024, loff[n]);
    };
    auto issue_k = [&](int t) { issue(K + kv_base, kring + ((t - t_lo) & 1) * TILE, t); };
    auto issue_v = [&](int t) { issue(V + kv_base, vring + ((t - t_lo) & 1) * TILE, t); };

    // Prologue: K(t_lo), V(t_lo).  Step t issues K(t+1), V(t+1) into the
    // slots of tile t-1, read for the last time in step t-1.  (Each key group
    // loads its own tiles.)
    if (t_lo < n_kt) {
        issue_k(t_lo);
        issue_v(t_lo);
    }

    f32x16 oacc[RB][D / 32];
    float m_use[RB];  // base of the exponent (log2 units), per row
    float l_run[RB];  // sum of bf16 weights relative to m_use (this lane's keys)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
        for (int db = 0; db < D / 32; ++db) oacc[rb][db] = f32x16{};
        m_use[rb] = -INFINITY;
        l_run[rb] = 0.f;
    }
    const bf16x2 ones = {(bf16)1.f, (bf16)1.f};

    const int xaddr = 4 * (lane ^ 32);  // half exchange
    uint32_t voff[2][D / 32];           // V^T read offsets within a tile
    pv_lane_offsets<D>(voff, lane);

    STile<BN, RB> s_cur;  // scores of the current tile
    // Step-0 address of this lane's K fragments in K slot 0 (see score_tile).
    const uint32_t ka0 = lds_u32(kring) + (uint32_t)(l32 * ROWB + ((hi ^ swz<CPR>(l32)) << 4));

    // Step t with PAR = (t - t_lo) & 1 known at compile time: K(t) and V(t)
    // sit in slot PAR.
    auto step = [&](int t, auto par) {
        constexpr int PAR = decltype(par)::value;
        const int j0 = t * BN;
        // K(t) and V(t), issued one step ago, must be complete in LDS (for
        // every wave's loads), and every wave must be done reading K(t-1) and
        // V(t-1), whose slots are refilled below.
        wait_vmem_all();
        __syncthreads();
        // The next tile's loads go out right after the barrier with 64-key
        // tiles (short steps need the lead), after this tile's score MFMAs
        // with 128-key tiles (measured +0.6-0.8% there, -1.5-2% with 64-key
        // tiles).
        constexpr bool kIssueAfterScores = BN >= 128;
        auto issue_next = [&]() {
            if (t + 1 < n_kt) {
                issue_k(t + 1);
                issue_v(t + 1);
            }
        };
        if (!kIssueAfterScores) issue_next();
        // Tiles above the diagonal or left of this wave's window, or a key
        // group's step past its last tile: nothing to do.
        if (t >= n_kt || !wave_live(j0)) {
            if (kIssueAfterScores) issue_next();
            return;
        }
        score_tile<D, BN, RB, PAR * TILE>(s_cur, ka0, qf);
        if (kIssueAfterScores) issue_next();

        // Per row block: element mask on tiles that cross the diagonal, a
        // window edge or the end of the keys.
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            // This block's rows see none of these keys: skip.
            if (j0 >= rb_kv_end[rb] || j0 + BN <= rb_kv_begin[rb]) continue;
            const int r0 = row0 + rb * 32;
            const int rlast = min(T_q - 1, r0 + 31);
            const bool need_mask = (j0 + BN > T_kv) || (CAUSAL && j0 + BN - 1 > r0 + off) ||
                                   (windowed && j0 < first_key(rlast));
            if (need_mask) {
                const int lim = CAUSAL ? min(T_kv - 1, r0 + l32 + off) : T_kv - 1;
                const int lo = windowed ? r0 + l32 + off - window + 1 : 0;
#pragma unroll
                for (int kb = 0; kb < BN / 32; ++kb) {
#pragma unroll
                    for (int j = 0; j < 16; ++j) {
                        const int key = j0 + kb * 32 + 8 * (j >> 2) + 4 * hi + (j & 3);
                        s_cur.acc[rb][kb][j] = (key <= lim && key >= lo) ? s_cur.acc[rb][kb][j] : -INFINITY;
                    }
                }
            }
        }

        // Weights 2^(score * c - base), rounded to bf16 in place (they are
        // the B operand of P V), and this lane's share of the row sum, taken
        // from the rounded weights.  A row block with no visible key in this
        // tile contributes nothing: its weights are zero.
        bf16x8 pb[RB][BN / 16];
        float psum[RB];
        auto weigh = [&]() {
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                const bool live = j0 < rb_kv_end[rb] && j0 + BN > rb_kv_begin[rb];
                const float m_sub = (m_use[rb] == -INFINITY) ? 0.f : m_use[rb];
                const float cc = live ? c : 0.f;
                const float msub = live ? m_sub : INFINITY;
                float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
                for (int kb = 0; kb < BN / 32; ++kb) {
#pragma unroll
                    for (int j = 0; j < 16; j += 2) {
                        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s_cur.acc[rb][kb][j], cc, -msub));
                        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s_cur.acc[rb][kb][j + 1], cc, -msub));
                        const bf16x2 pp = {(bf16)p0, (bf16)p1};
                        if (j & 2) ps1 = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, ps1, false);
                        else ps0 = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, ps0, false);
                        pb[rb][kb * 2 + (j >> 3)][j & 7] = pp[0];
                        pb[rb][kb * 2 + (j >> 3)][(j & 7) + 1] = pp[1];
                    }
                }
                psum[rb] = ps0 + ps1;
            }
        };
        weigh();

        // The base of a row stays where it is as long as every weight is
        // small enough: no row maximum is taken on that path.  The base moves
        // (to the row's exact maximum, both halves of the row exchanged via
        // lane ^ 32) only when some lane's share of a row sum exceeds 2^16
        // (a weight grew past 2^16 / (BN / 2), or overflowed to infinity), or
        // when a row has no base yet; the weights are then recomputed.  So
        // weights stay below 2^16 and the fp32 accumulators far from
        // overflow; O / l is the same for any base.
        bool rebase = false;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) rebase |= (m_use[rb] == -INFINITY) || !(psum[rb] <= kSumGuard);
        if (__any(rebase)) {
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                if (j0 >= rb_kv_end[rb] || j0 + BN <= rb_kv_begin[rb]) continue;
                // This lane's maximum: two chains of three-input maxima.
                float mxa = -INFINITY, mxb = -INFINITY;
#pragma unroll
                for (int kb = 0; kb < BN / 32; ++kb) {
#pragma unroll
                    for (int j = 0; j < 16; j += 4) {
                        mxa = fmaxf(fmaxf(mxa, s_cur.acc[rb][kb][j]), s_cur.acc[rb][kb][j + 1]);
                        mxb = fmaxf(fmaxf(mxb, s_cur.acc[rb][kb][j + 2]), s_cur.acc[rb][kb][j + 3]);
                    }
                }
                const float mx = fmaxf(mxa, mxb);
                const float m_row = fmaxf(mx, swap_halves(mx, xaddr)) * c;  // -inf: no visible key yet
                const float m_t = fmaxf(m_use[rb], m_row);
                // While a row has no base it has accumulated nothing, so
                // alpha = 0 (or 1 when it still has no key) is exact.
                const float alpha = (m_t == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_use[rb] - m_t);
                l_run[rb] *= alpha;
#pragma unroll
                for (int db = 0; db < D / 32; ++db) {
#pragma unroll
                    for (int j = 0; j < 16; ++j) oacc[rb][db][j] *= alpha;
                }
                m_use[rb] = m_t;
            }
            weigh();
        }
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) l_run[rb] += psum[rb];

        // O^T += V^T P^T for tile t.
        const uint32_t vbase = lds_u32(vring + PAR * TILE);
        uint32_t va[2][D / 32];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int db = 0; db < D / 32; ++db) va[h][db] = vbase + voff[h][db];
        }
        // Raised wave priority while the P V MFMAs issue: the other wave of
        // the SIMD then fills the matrix-core gaps with its own score or
        // vector work instead of delaying these (+1-3% measured).
        __builtin_amdgcn_s_setprio(1);
        pv_tile<D, BN / 16, RB>(oacc, pb, va);
        __builtin_amdgcn_s_setprio(0);
    };
    // Every key group runs n_steps steps (one barrier per step for all waves).
    for (int i = 0; i < n_steps; i += 2) {
        step(t_lo + i, std::integral_constant<int, 0>{});
        if (i + 1 < n_steps) step(t_lo + i + 1, std::integral_constant<int, 1>{});
    }

    if constexpr (KSPLIT == 2) {
        // Merge the second key group's state into the first's: per lane
        // (D / 2 partial outputs, base, row sum) through LDS, now free.
        constexpr int XS = D / 2 + 2;  // floats per lane
        float* xch = reinterpret_cast<float*>(smem) + (size_t)(wave * 64 + lane) * XS;
        const float l_mine = l_run[0] + swap_halves(l_run[0], xaddr);
        __syncthreads();
        if (kg == 1) {
#pragma unroll
            for (int db = 0; db < D / 32; ++db) {
#pragma unroll
                for (int j = 0; j < 16; ++j) xch[db * 16 + j] = oacc[0][db][j];
            }
            xch[D / 2] = m_use[0];
            xch[D / 2 + 1] = l_mine;
        }
        __syncthreads();
        if (kg == 1) return;
        const float m_b = xch[D / 2], l_b = xch[D / 2 + 1];
        const float m_a = m_use[0];
        const float mm = fmaxf(m_a, m_b);
        const float a = m_a == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_a - mm);
        const float bw = m_b == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_b - mm);
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
#pragma unroll
            for (int j = 0; j < 16; ++j) oacc[0][db][j] = oacc[0][db][j] * a + xch[db * 16 + j] * bw;
        }
        // the epilogue below adds the two halves of the row sum again
        l_run[0] = l_mine * a * 0.5f + l_b * bw * 0.5f;
    }

    // Epilogue: O = O_acc / l, rounded once to bf16.  Rows past T_q fall
    // outside the buffer range and their stores are dropped.  A row that
    // sees no key (possible only in a packed batch) gets O = 0.
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const float l_tot = l_run[rb] + swap_halves(l_run[rb], xaddr);
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        const int my_row = row0 + rb * 32 + l32;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                bf16x4 w;
#pragma unroll
                for (int r = 0; r < 4; ++r) w[r] = (bf16)(oacc[rb][db][4 * g4 + r] * inv);
                buf_store_b64(__builtin_bit_cast(u32x2, w), rO,
                              (uint32_t)(my_row * SQ + db * 32 + 8 * g4 + 4 * hi) * 2);
            }
        }
    }
}

template <int D, bool CAUSAL, bool VARLEN, int RB, int BN, int WAVES, int WPE, int KSPLIT = 1>
hipError_t launch_cfg(const PrefillArgs& a, hipStream_t s) {
    constexpr int BM = 32 * RB * WAVES / KSPLIT;
    const int n_qt = (a.T_q + BM - 1) / BM;
    const long long grid = (long long)a.B * a.H_q * n_qt;
    return launch_kernel(prefill_bf16_kernel<D, CAUSAL, VARLEN, RB, BN, WAVES, WPE, KSPLIT>,
                         dim3((unsigned)grid), dim3(64 * WAVES), 0, s, static_cast<const bf16*>(a.q),
                         static_cast<const bf16*>(a.k), static_cast<const bf16*>(a.v),
                         static_cast<bf16*>(a.o), a.B, a.H_q, a.H_kv, a.T_q, a.T_kv, n_qt, a.c_log2,
                         a.neg_q, a.window, a.cu_q, a.cu_k);
}

// Long sequences with at least two 256-row workgroups per CU: 8 waves and
// 128-key tiles, one workgroup per CU (one K/V tile in LDS serves 256 rows;
// 128 KiB of LDS; twice the keys per barrier than 64-key tiles, +3%).
// Otherwise 4 waves and 64-key tiles, two workgroups per CU (64 KiB each):
// with short sequences the per-workgroup start-up and the diagonal tiles
// weigh more, and 128-row workgroups were measured faster (T = 512: 528 vs
// 446 TFLOP/s; T = 1024: 710 vs 650; equal at T = 4096).
template <int D, bool CAUSAL, bool VARLEN>
hipError_t launch_one(const PrefillArgs& a, hipStream_t s) {
    const long long wg_big = (long long)a.B * a.H_q * ((a.T_q + 255) / 256);
    const long long rows_per_seq = VARLEN ? a.total_q / (a.B > 0 ? a.B : 1) : a.T_q;
    const bool big = wg_big >= 512 && rows_per_seq >= 4096;
    if (big) return launch_cfg<D, CAUSAL, VARLEN, 1, 128, 8, 2>(a, s);
    // Short problems whose 128-row workgroups all fit on the GPU at once
    // (D = 64: 512 of them, two per CU; D = 128: 256): 8 waves in two key
    // groups halve the longest chain of steps.  (A packed batch sizes the
    // grid by its longest sequence, as dense problems by T_q.)
    const long long wg4 = (long long)a.B * a.H_q * ((a.T_q + 127) / 128);
    if (a.T_kv >= 128 && wg4 <= (D == 64 ? 512 : 256))
        return launch_cfg<D, CAUSAL, VARLEN, 1, 64, 8, D == 64 ? 4 : 2, 2>(a, s);
    return launch_cfg<D, CAUSAL, VARLEN, 1, 64, 4, 2>(a, s);
}

template <int D>
hipError_t launch_d(const PrefillArgs& a, hipStream_t s) {
    if (a.cu_q) return a.causal ? launch_one<D, true, true>(a, s) : launch_one<D, false, true>(a, s);
    return a.causal ? launch_one<D, true, false>(a, s) : launch_one<D, false, false>(a, s);
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t s) {
    return a.D == 128 ? launch_d<128>(a, s) : launch_d<64>(a, s);
}

}  // namespace attn
