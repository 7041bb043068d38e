// bf16 attention forward for decode (one query token per sequence), gfx950.
//
// Decode is a vector against the whole KV cache and is bound by reading K
// and V from HBM (learn-cuda-from-scratch Ch. 11 "Attention", section
// 11.8.2; AIInfraGuide "3.3 Self-Attention机制深入理解", section 11.2).
// Two passes:
//
//   1. split pass: the keys of each (batch, kv head) are cut into n_splits
//      contiguous ranges.  One wave owns one range and all query heads that
//      read this kv head (up to 32 per wave), so K and V are read from HBM
//      once for the whole group (the GQA saving of Ch. 11 section 11.8.1).
//      It keeps the online-softmax state (exponent base m in log2 units, sum
//      l, unnormalised output) and writes it to the workspace.
//   2. combine pass: per (batch, q head) the split states are merged with the
//      block-merge rule of AIInfraGuide section 12.3:
//      m = max m_s, l = sum l_s 2^(m_s - m), O = sum O_s 2^(m_s - m) / l.
//      With a single split (enough (batch, kv head) groups to fill the GPU)
//      the split pass normalises and writes O itself; no workspace is used.
//
// The split pass uses the prefill kernel's MFMA layout with the query heads
// of the group as the 32 MFMA columns: S^T = K Q^T on
// v_mfma_f32_32x32x16_bf16, then O^T += V^T P^T with the V^T operand read by
// ds_read_b64_tr_b16 (issued as inline assembly, see ds_read_tr16_asm).
// Each wave streams 32-key tiles of K and V from HBM
// straight into its own LDS ring of kStages tiles with 16-byte buffer loads
// (each 1 KiB load covers four whole rows), keeping kStages - 1 tiles in
// flight while it consumes one; waves never synchronise with each other.
// The cache is read exactly once per call, so these loads carry the
// non-temporal hint (6.15 -> 6.7 TB/s contiguous, 5.9 -> 6.5 paged).
//
// Paged KV cache (the serving form; Ch. 11 page, section 11.11 on KV-cache
// pages of 16 tokens and the block table that maps (request, token / 16) to
// a physical block): K and V live in pools of pages [num_pages][H_kv]
// [page_size][D]; token j of sequence b is row j % page_size of page
// block_table[b][j / page_size].  The split kernel is the same; only the
// tile loads change: every 1 KiB load covers rows of one page, addressed
// through a buffer resource built for that page (so the pool may be of any
// size, rows past the sequence's length read as zero, and a block id outside
// the pool reads as a page of zeros instead of faulting).  The block ids of
// 64 consecutive pages are held one per lane and picked with v_readlane.
#include "launch.h"

namespace attn {
namespace {

constexpr int kBN = 32;     // keys per tile
// LDS ring depth per wave: two tiles in flight while one is consumed (with
// the non-temporal loads: +1.5% contiguous, +1% paged over a 2-deep ring).
constexpr int kStages = 3;

// Wait until tile t of the ring has landed: `ahead` later tiles (PER loads
// each) may still be in flight.  Loads complete in issue order.
template <int PER>
__device__ inline void wait_tiles_ahead(int ahead) {
    static_assert(3 * PER < 64, "vmcnt is 6 bits");
    switch (ahead) {
        case 0: wait_vmem_le<0>(); break;
        case 1: wait_vmem_le<PER>(); break;
        case 2: wait_vmem_le<2 * PER>(); break;
        default: wait_vmem_le<3 * PER>(); break;
    }
}

template <int D, bool PAGED>
__global__ __launch_bounds__(64) void decode_split_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    bf16* __restrict__ O, float* __restrict__ ws_o, float* __restrict__ ws_ml, int H_q, int H_kv,
    int T_kv, int n_splits, int kps, int n_hb, float c, int neg_q, PagedKV pg) {
    constexpr int CPR = D / 8;
    constexpr int ROWB = D * 2;
    constexpr int TILE = kBN * ROWB;  // bytes of one K or V tile
    constexpr int NLD = TILE / 1024;  // 1 KiB loads per tile and operand
    static_assert(NLD * 1024 == TILE && kStages - 2 <= 3, "vmcnt budget");

    __shared__ __attribute__((aligned(1024))) unsigned char smem[kStages * 2 * TILE];

    const int lane = threadIdx.x;
    const int l32 = lane & 31;
    const int hi = lane >> 5;

    const int gw = blockIdx.x;
    const int split = gw % n_splits;
    const int rest = gw / n_splits;
    const int hb = rest % n_hb;
    const int unit = rest / n_hb;  // (batch, kv head)
    const int b = unit / H_kv;
    const int hk = unit - b * H_kv;
    const int G = H_q / H_kv;
    const int gi = hb * 32 + l32;  // query head within the group (MFMA column)
    const bool valid = gi < G;
    const int hq = hk * G + gi;

    // Keys of this sequence: T_kv, or its own length in the paged form
    // (clamped to the block table's capacity T_kv; 0 gives O = 0).
    int seq_len = T_kv;
    if constexpr (PAGED) seq_len = min(max(pg.seq_lens[b], 0), T_kv);
    const int k0 = split * kps;
    const int k1 = min(seq_len, k0 + kps);
    const int n_t = k1 > k0 ? (k1 - k0 + kBN - 1) / kBN : 0;

    // Contiguous cache: this split's keys only; loads past k1 read as zero.
    const uint32_t split_bytes = PAGED ? 0u : (uint32_t)(k1 - k0) * ROWB;
    const size_t split_base = PAGED ? 0 : ((size_t)unit * T_kv + k0) * D;
    const auto rK = make_rsrc(K + split_base, split_bytes);
    const auto rV = make_rsrc(V + split_base, split_bytes);

    // Paged cache: block ids of pages [id_base, id_base + 64), one per lane.
    int id_base = -(1 << 30), ids = 0;
    const int page_size = 1 << pg.page_shift;
    auto block_of = [&](int page) {
        if (page - id_base >= 64 || page < id_base) {
            // Rare (every 64 pages): the wait also drains the tile loads.
            const auto rT = make_rsrc(pg.block_table + (size_t)b * pg.max_pages,
                                      (uint32_t)pg.max_pages * 4);
            id_base = page;
            ids = __builtin_amdgcn_raw_buffer_load_b32(rT, (page + lane) * 4, 0, 0);
            wait_vmem_all();
        }
        return __builtin_amdgcn_readlane(ids, page - id_base);
    };
    // Rows [page * page_size, seq_len) of one page of a pool.
    auto page_rsrc = [&](const bf16* pool, int page, int blk) {
        const int rows = min(page_size, seq_len - (page << pg.page_shift));
        const bool ok = rows > 0 && (unsigned)blk < (unsigned)pg.num_pages;
        const bf16* base = pool + ((size_t)(ok ? blk : 0) * H_kv + hk) * ((size_t)page_size * D);
        return make_rsrc(base, ok ? (uint32_t)rows * ROWB : 0u);
    };

    auto issue = [&](int t) {
        unsigned char* kst = smem + (t % kStages) * 2 * TILE;
        unsigned char* vst = kst + TILE;
        if constexpr (PAGED) {
            // A 32-key tile spans one page, or two when page_size == 16.
            const int key_t = k0 + t * kBN;
            const int pa = key_t >> pg.page_shift, pb = (key_t + 16) >> pg.page_shift;
            const int ba = block_of(pa), bb = block_of(pb);
            const auto kA = page_rsrc(K, pa, ba), vA = page_rsrc(V, pa, ba);
            const auto kB = page_rsrc(K, pb, bb), vB = page_rsrc(V, pb, bb);
#pragma unroll
            for (int n = 0; n < NLD; ++n) {
                const int p = n * 64 + lane;
                const int row = p / CPR;
                const int logical = (p % CPR) ^ swz<CPR>(row);
                const bool second = ((key_t + n * (64 / CPR)) >> pg.page_shift) != pa;
                const uint32_t boff =
                    (uint32_t)((key_t + row) & (page_size - 1)) * ROWB + logical * 16;
                buf_load_lds16_nt(second ? kB : kA, kst + n * 1024, boff);
                buf_load_lds16_nt(second ? vB : vA, vst + n * 1024, boff);
            }
        } else {
#pragma unroll
            for (int n = 0; n < NLD; ++n) {
                const int p = n * 64 + lane;
                const int row = p / CPR;
                const int logical = (p % CPR) ^ swz<CPR>(row);
                const uint32_t boff = (uint32_t)(t * kBN + row) * ROWB + logical * 16;
                buf_load_lds16_nt(rK, kst + n * 1024, boff);
                buf_load_lds16_nt(rV, vst + n * 1024, boff);
            }
        }
    };

#pragma unroll
    for (int t = 0; t < kStages - 1; ++t)
        if (t < n_t) issue(t);

    // Query heads of this group as MFMA columns; heads past the group read as
    // zero.  A negative scale is folded into Q's sign, so c > 0.
    const int g_rows = min(32, G - hb * 32);
    const auto rQ = make_rsrc(Q + (size_t)(b * H_q + hk * G + hb * 32) * D, (uint32_t)g_rows * ROWB);
    bf16x8 qf[D / 16];
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
        u32x4 w = buf_load_b128(rQ, (uint32_t)(l32 * D + 16 * s + 8 * hi) * 2);
        if (neg_q) w ^= 0x80008000u;
        qf[s] = __builtin_bit_cast(bf16x8, w);
    }

    f32x16 oacc[1][D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) oacc[0][db] = f32x16{};
    float m_use = -INFINITY;
    float l_run = 0.f;
    const bf16x2 ones = {(bf16)1.f, (bf16)1.f};

    const int xaddr = 4 * (lane ^ 32);
    uint32_t voff[2][D / 32];  // V^T read offsets within a tile
    pv_lane_offsets<D>(voff, lane);

    for (int t = 0; t < n_t; ++t) {
        // The Q loads were issued after the first tiles, so they are covered
        // by the same counter.
        wait_tiles_ahead<2 * NLD>(min(kStages - 2, n_t - 1 - t));
        if (t + kStages - 1 < n_t) issue(t + kStages - 1);  // refills the stage read at t - 1

        const unsigned char* kst = smem + (t % kStages) * 2 * TILE;
        const unsigned char* vst = kst + TILE;

        f32x16 sacc = f32x16{};
        {
            const int key = l32;
            const unsigned char* krow = kst + key * ROWB;
            const int sw = swz<CPR>(key);
#pragma unroll
            for (int s = 0; s < D / 16; ++s) {
                const bf16x8 a = *reinterpret_cast<const bf16x8*>(krow + (((2 * s + hi) ^ sw) * 16));
                sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], sacc, 0, 0, 0);
            }
        }
        const int jr = t * kBN;  // first key of the tile, relative to k0
        if (k0 + jr + kBN > k1) {
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int key = jr + 8 * (j >> 2) + 4 * hi + (j & 3);
                sacc[j] = (k0 + key < k1) ? sacc[j] : -INFINITY;
            }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int j = 0; j < 16; j += 2) mx = fmaxf(mx, fmaxf(sacc[j], sacc[j + 1]));
        mx = fmaxf(mx, swap_halves(mx, xaddr));
        const float m_new = mx * c;
        if (__any(m_new > m_use + 8.f)) {
            const float m_t = fmaxf(m_use, m_new);
            const float alpha = (m_t == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_use - m_t);
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < D / 32; ++db) {
#pragma unroll
                for (int j = 0; j < 16; ++j) oacc[0][db][j] *= alpha;
            }
            m_use = m_t;
        }
        const float m_sub = (m_use == -INFINITY) ? 0.f : m_use;

        bf16x8 pb[1][2];
        float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
        for (int j = 0; j < 16; j += 2) {
            const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[j], c, -m_sub));
            const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[j + 1], c, -m_sub));
            const bf16x2 pp = {(bf16)p0, (bf16)p1};
            if (j & 2) ps1 = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, ps1, false);
            else ps0 = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, ps0, false);
            pb[0][j >> 3][j & 7] = pp[0];
            pb[0][j >> 3][(j & 7) + 1] = pp[1];
        }
        l_run += ps0 + ps1;

        // O^T += V^T P^T over the tile's two key steps.  With a contiguous
        // cache this wave's tiles in flight are drained first (with plain
        // loads 6.1 TB/s against 5.9 without; with the non-temporal loads
        // and a 3-deep ring: 6.8 against 6.5); with pages they are left in
        // flight (5.8 against 5.3 TB/s with plain loads): the scattered
        // 4 KiB page reads need the overlap.
        if constexpr (!PAGED) wait_vmem_all();
        const uint32_t vbase = lds_u32(vst);
        uint32_t va[2][D / 32];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int db = 0; db < D / 32; ++db) va[h][db] = vbase + voff[h][db];
        }
        pv_tile<D, kBN / 16, 1>(oacc, pb, va);
    }

    const float l_tot = l_run + swap_halves(l_run, xaddr);
    if (!valid) return;
    const size_t row = (size_t)(b * H_q + hq);
    if (n_splits == 1) {
        // The single split covers every key: normalise and write O directly
        // (an empty paged sequence has l = 0 and gets O = 0).
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        bf16* orow = O + row * D + 4 * hi;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                bf16x4 w;
#pragma unroll
                for (int r = 0; r < 4; ++r) w[r] = (bf16)(oacc[0][db][4 * g4 + r] * inv);
                *reinterpret_cast<bf16x4*>(orow + db * 32 + 8 * g4) = w;
            }
        }
        return;
    }
    const size_t idx = row * n_splits + split;
    float* op = ws_o + idx * D + 4 * hi;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            const f32x4 w = {oacc[0][db][4 * g4], oacc[0][db][4 * g4 + 1], oacc[0][db][4 * g4 + 2],
                             oacc[0][db][4 * g4 + 3]};
            *reinterpret_cast<f32x4*>(op + db * 32 + 8 * g4) = w;
        }
    }
    if (hi == 0) {
        ws_ml[2 * idx] = m_use;
        ws_ml[2 * idx + 1] = l_tot;
    }
}

// Four waves per (batch, q head): merge the split states and write O.  Lane
// (split group g = 4 * wave + lane / 16, feature group fq = lane % 16)
// merges splits g, g + 16, g + 32, ... for features fq * D/16 ... with the
// online form of the merge rule (running base, sum and output), four
// splits' loads in flight at a time; the four split groups of a wave are
// merged across lanes (two exchanges), the four waves' states through LDS,
// and wave 0 writes O.  (One wave per row took twice as long with 125
// splits: its lanes walked the splits in twice as many dependent rounds.)
constexpr int kCombineWaves = 4;  // waves per output row in the combine pass

template <int D>
__global__ __launch_bounds__(64 * kCombineWaves) void decode_combine_kernel(const float* __restrict__ ws_o,
                                                                           const float* __restrict__ ws_ml,
                                                                           bf16* __restrict__ O, int n_splits) {
    constexpr int FPL = D / 16;  // features per lane
    constexpr int NG = 4 * kCombineWaves;  // split groups of the row
    __shared__ float xs[kCombineWaves][16][FPL + 2];
    const size_t row = blockIdx.x;
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int sg = lane >> 4, fq = lane & 15;
    const int gsg = wave * 4 + sg;  // this lane's split group
    const float* ml = ws_ml + row * n_splits * 2;
    const float* op = ws_o + row * n_splits * D + fq * FPL;
    float m = -INFINITY, L = 0.f, acc[FPL];
#pragma unroll
    for (int f = 0; f < FPL; ++f) acc[f] = 0.f;
    // merge a state (ms, ls, o) into (m, L, acc); a state with base -inf (an
    // empty split, or a group with no split) carries nothing
    auto merge = [&](float ms, float ls, const float (&o)[FPL]) {
        if (ms == -INFINITY) return;
        const float mn = fmaxf(m, ms);
        const float a = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - mn);
        const float w = __builtin_amdgcn_exp2f(ms - mn);
        L = L * a + ls * w;
#pragma unroll
        for (int f = 0; f < FPL; ++f) acc[f] = acc[f] * a + o[f] * w;
        m = mn;
    };
    constexpr int U = 4;  // splits per lane in flight
    for (int s0 = gsg; s0 < n_splits; s0 += NG * U) {
        float ms[U], ls[U];
        float o[U][FPL];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int sp = s0 + NG * u;
            ms[u] = -INFINITY;
            ls[u] = 0.f;
            if (sp < n_splits) {
                ms[u] = ml[2 * sp];
                ls[u] = ml[2 * sp + 1];
#pragma unroll
                for (int c = 0; c < FPL / 4; ++c) {
                    const f32x4 v = *reinterpret_cast<const f32x4*>(op + (size_t)sp * D + 4 * c);
                    o[u][4 * c] = v[0];
                    o[u][4 * c + 1] = v[1];
                    o[u][4 * c + 2] = v[2];
                    o[u][4 * c + 3] = v[3];
                }
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) merge(ms[u], ls[u], o[u]);
    }
    // merge the four split groups of the wave: lanes lane ^ 16, then lane ^ 32
#pragma unroll
    for (int x = 16; x <= 32; x <<= 1) {
        const float m2 = __shfl_xor(m, x), L2 = __shfl_xor(L, x);
        float o2[FPL];
#pragma unroll
        for (int f = 0; f < FPL; ++f) o2[f] = __shfl_xor(acc[f], x);
        merge(m2, L2, o2);
    }
    // then the waves' states, through LDS, into wave 0
    if (sg == 0 && wave > 0) {
#pragma unroll
        for (int f = 0; f < FPL; ++f) xs[wave][fq][f] = acc[f];
        xs[wave][fq][FPL] = m;
        xs[wave][fq][FPL + 1] = L;
    }
    __syncthreads();
    if (wave != 0 || sg != 0) return;
#pragma unroll
    for (int w = 1; w < kCombineWaves; ++w) {
        float o2[FPL];
#pragma unroll
        for (int f = 0; f < FPL; ++f) o2[f] = xs[w][fq][f];
        merge(xs[w][fq][FPL], xs[w][fq][FPL + 1], o2);
    }
    // every split empty (a paged sequence of length 0): L = 0, O = 0
    const float inv = L > 0.f ? 1.f / L : 0.f;
    bf16* orow = O + row * D + fq * FPL;
#pragma unroll
    for (int g4 = 0; g4 < FPL / 4; ++g4) {
        bf16x4 w;
#pragma unroll
        for (int q = 0; q < 4; ++q) w[q] = (bf16)(acc[4 * g4 + q] * inv);
        *reinterpret_cast<bf16x4*>(orow + 4 * g4) = w;
    }
}

template <int D, bool PAGED>
hipError_t launch_d(const DecodeArgs& a, hipStream_t s) {
    const int G = a.H_q / a.H_kv;
    const int n_hb = (G + 31) / 32;
    const long long waves = (long long)a.B * a.H_kv * n_hb * a.n_splits;
    hipError_t e = launch_kernel(decode_split_kernel<D, PAGED>, dim3((unsigned)waves), dim3(64), 0, s,
                                 static_cast<const bf16*>(a.q), static_cast<const bf16*>(a.k),
                                 static_cast<const bf16*>(a.v), static_cast<bf16*>(a.o), a.ws_o, a.ws_ml,
                                 a.H_q, a.H_kv, a.T_kv, a.n_splits, a.keys_per_split, n_hb, a.c_log2,
                                 a.neg_q, a.paged);
    if (e != hipSuccess || a.n_splits == 1) return e;
    const long long rows = (long long)a.B * a.H_q;
    return launch_kernel(decode_combine_kernel<D>, dim3((unsigned)rows), dim3(64 * kCombineWaves), 0, s,
                         static_cast<const float*>(a.ws_o), static_cast<const float*>(a.ws_ml),
                         static_cast<bf16*>(a.o), a.n_splits);
}

}  // namespace

hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t s) {
    if (a.paged.block_table) return a.D == 128 ? launch_d<128, true>(a, s) : launch_d<64, true>(a, s);
    return a.D == 128 ? launch_d<128, false>(a, s) : launch_d<64, false>(a, s);
}

}  // namespace attn
