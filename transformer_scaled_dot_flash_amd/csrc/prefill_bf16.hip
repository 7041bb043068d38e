// bf16 attention forward, prefill shape (any T_q), for gfx950.
//
// Method: FlashAttention-style tiling with online softmax (AIInfraGuide
// "3.3 Self-Attention机制深入理解", sections 7.3, 12.2, 12.3): each
// workgroup owns 128 query rows of one (batch, q head), walks the key/value
// tiles of its kv head, keeps a running row maximum m, a running exponential
// sum l and an unnormalised output accumulator in registers, rescales them
// when m grows, and divides by l once at the end.  Scores and weights never
// leave the chip.
//
// gfx950 mapping:
//   * 4 waves x 32 query rows.  Each wave computes S^T = K * Q^T for 32 keys
//     at a time with v_mfma_f32_32x32x16_bf16, so the accumulator layout puts
//     one query row in each lane column and 16 keys in each lane: the row
//     maximum and row sum are in-lane, plus a single exchange with lane^32.
//   * The same layout is the B operand of O^T = V^T * P^T: the weights are
//     converted to bf16 in place and never move between lanes.  V is stored
//     transposed in LDS (key-contiguous per feature) so the A operand of the
//     P*V product is two 8-byte LDS reads per lane.
//   * K and V tiles come from HBM with 16-byte loads, each row of a tile read
//     contiguously, and are double-buffered in LDS: the next tile is in
//     flight in registers while the current one is consumed.  XOR swizzles
//     keep the LDS reads and writes free of bank conflicts without padding.
//   * Causal: key tiles wholly above the diagonal are never visited (per
//     workgroup) or skipped (per wave); only tiles that cross the diagonal or
//     the end of the keys pay for the element mask (Ch. 11 "Attention" page,
//     section 11.8.3), using exact tile bounds.
//   * Workgroups are ordered heaviest query tile first (causal work grows
//     along the sequence) and, when the kv-head count allows, all workgroups
//     of one kv head are placed on one XCD so its K/V stay in that XCD's L2.
#include "kernel_common.h"

namespace attn {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBM = 32 * kWaves;  // query rows per workgroup

struct TileCoord {
    int qt, b, hq, hk;
};

// Workgroup id -> (query tile, batch, q head, kv head).
__device__ inline TileCoord map_tile(int id, int B, int H_q, int H_kv, int n_qt, bool causal) {
    const int G = H_q / H_kv;
    const int units = B * H_kv;  // (batch, kv head) pairs
    int qt_rev, unit, g;
    if ((units & 7) == 0) {
        // Dispatch sends workgroup id to XCD (id mod 8).  Give each XCD a
        // contiguous block of kv heads; within it, heaviest query tile first.
        const int xcd = id & 7;
        const int slot = id >> 3;
        const int upx = units >> 3;
        const int per = upx * G;
        qt_rev = slot / per;
        const int rem = slot - qt_rev * per;
        const int u = rem / G;
        unit = xcd * upx + u;
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

// Transposed-V swizzle: feature row d stores its 4-key group g at g ^ vswz(d).
__device__ inline int vswz(int d) { return (d ^ (d >> 3)) & 15; }

__device__ inline uint32_t pack_lo(uint32_t a, uint32_t b) { return (a & 0xffffu) | (b << 16); }
__device__ inline uint32_t pack_hi(uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xffff0000u); }

template <int D, int BN, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void prefill_bf16_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    bf16* __restrict__ O, int B, int H_q, int H_kv, int T_q, int T_kv, int n_qt, float scale_log2) {
    constexpr int CPR = D / 8;          // 16-byte chunks per row
    constexpr int KSW = CPR - 1;        // K chunk swizzle mask
    constexpr int STAGE = 2 * BN * D;   // bf16 elements per LDS stage (K + V^T)
    constexpr int NK = BN * CPR / kThreads;
    constexpr int NVQ = (BN / 4) * CPR / kThreads;
    static_assert(NK * kThreads == BN * CPR, "K tile must split evenly over threads");
    static_assert(NVQ * kThreads == (BN / 4) * CPR, "V tile must split evenly over threads");
    static_assert(BN % 32 == 0 && BN / 4 >= 16, "key tile");

    __shared__ __attribute__((aligned(16))) bf16 smem[2 * STAGE];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int hi = lane >> 5;

    const TileCoord tc = map_tile(blockIdx.x, B, H_q, H_kv, n_qt, CAUSAL);
    const uint32_t q_bytes = (uint32_t)T_q * D * 2;
    const uint32_t kv_bytes = (uint32_t)T_kv * D * 2;
    const auto rQ = make_rsrc(Q + (size_t)(tc.b * H_q + tc.hq) * T_q * D, q_bytes);
    const auto rK = make_rsrc(K + (size_t)(tc.b * H_kv + tc.hk) * T_kv * D, kv_bytes);
    const auto rV = make_rsrc(V + (size_t)(tc.b * H_kv + tc.hk) * T_kv * D, kv_bytes);
    const auto rO = make_rsrc(O + (size_t)(tc.b * H_q + tc.hq) * T_q * D, q_bytes);

    const int off = T_kv - T_q;  // bottom-right causal alignment
    const int q0 = tc.qt * kBM;
    const int row0 = q0 + wave * 32;
    const int my_row = row0 + l32;

    // Q fragment: B operand of S^T = K Q^T (column = query row, 8 features).
    // Rows past T_q read as zero (buffer range check).
    bf16x8 qf[D / 16];
#pragma unroll
    for (int s = 0; s < D / 16; ++s)
        qf[s] = __builtin_bit_cast(bf16x8, buf_load_b128(rQ, (uint32_t)(my_row * D + 16 * s + 8 * hi) * 2));

    // Key ranges.
    const int last_row = min(T_q, q0 + kBM) - 1;
    const int kv_end = CAUSAL ? min(T_kv, last_row + off + 1) : T_kv;
    const int n_kt = (kv_end + BN - 1) / BN;
    const int wave_last = min(T_q - 1, row0 + 31);
    const int wave_kv_end = (row0 >= T_q) ? 0 : (CAUSAL ? min(T_kv, wave_last + off + 1) : T_kv);

    // Keys past T_kv read as zero (buffer range check) and are masked.
    u32x4 kr[NK];
    u32x4 vr[NVQ][4];

    auto load_tile = [&](int j0) {
#pragma unroll
        for (int i = 0; i < NK; ++i) {
            const int c = tid + i * kThreads;
            const int row = c / CPR, ch = c % CPR;
            kr[i] = buf_load_b128(rK, (uint32_t)((j0 + row) * D + ch * 8) * 2);
        }
#pragma unroll
        for (int i = 0; i < NVQ; ++i) {
            const int u = tid + i * kThreads;
            const int ch = u % CPR, kq = u / CPR;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                vr[i][r] = buf_load_b128(rV, (uint32_t)((j0 + 4 * kq + r) * D + ch * 8) * 2);
        }
    };

    auto store_tile = [&](int buf) {
        bf16* ks = smem + buf * STAGE;
        bf16* vt = ks + BN * D;
#pragma unroll
        for (int i = 0; i < NK; ++i) {
            const int c = tid + i * kThreads;
            const int row = c / CPR, ch = c % CPR;
            *reinterpret_cast<u32x4*>(ks + row * D + ((ch ^ (row & KSW)) * 8)) = kr[i];
        }
#pragma unroll
        for (int i = 0; i < NVQ; ++i) {
            const int u = tid + i * kThreads;
            const int ch = u % CPR, kq = u / CPR;
            const u32x4 w0 = vr[i][0], w1 = vr[i][1], w2 = vr[i][2], w3 = vr[i][3];
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                // features ch*8 + 2w (low halves) and ch*8 + 2w + 1 (high halves)
                const int d0 = ch * 8 + 2 * w;
                const int d1 = d0 + 1;
                const u32x2 lo = {pack_lo(w0[w], w1[w]), pack_lo(w2[w], w3[w])};
                const u32x2 hi2 = {pack_hi(w0[w], w1[w]), pack_hi(w2[w], w3[w])};
                *reinterpret_cast<u32x2*>(vt + d0 * BN + ((kq ^ vswz(d0)) * 4)) = lo;
                *reinterpret_cast<u32x2*>(vt + d1 * BN + ((kq ^ vswz(d1)) * 4)) = hi2;
            }
        }
    };

    f32x16 oacc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) oacc[db] = f32x16{};
    float m_run = -INFINITY;
    float l_run = 0.f;

    if (n_kt > 0) {
        load_tile(0);
        store_tile(0);
    }
    __syncthreads();

    for (int t = 0; t < n_kt; ++t) {
        const int j0 = t * BN;
        const bool has_next = t + 1 < n_kt;
        if (has_next) load_tile(j0 + BN);

        if (j0 < wave_kv_end) {
            const bf16* ks = smem + (t & 1) * STAGE;
            const bf16* vt = ks + BN * D;

            // S^T tile: rows = keys, columns = this wave's 32 query rows.
            f32x16 sacc[BN / 32];
#pragma unroll
            for (int kb = 0; kb < BN / 32; ++kb) {
                sacc[kb] = f32x16{};
                const int key = kb * 32 + l32;
                const bf16* krow = ks + key * D;
#pragma unroll
                for (int s = 0; s < D / 16; ++s) {
                    const int ch = (2 * s + hi) ^ (key & KSW);
                    const bf16x8 a = *reinterpret_cast<const bf16x8*>(krow + ch * 8);
                    sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], sacc[kb], 0, 0, 0);
                }
            }

            // Scale into log2 units, mask only where the tile needs it.
            const bool need_mask = (j0 + BN > T_kv) || (CAUSAL && j0 + BN - 1 > row0 + off);
            const int lim = CAUSAL ? min(T_kv - 1, my_row + off) : T_kv - 1;
            float mx = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < BN / 32; ++kb) {
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    float x = sacc[kb][j] * scale_log2;
                    if (need_mask) {
                        const int key = j0 + kb * 32 + 8 * (j >> 2) + 4 * hi + (j & 3);
                        x = key <= lim ? x : -INFINITY;
                    }
                    sacc[kb][j] = x;
                    mx = fmaxf(mx, x);
                }
            }
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float m_new = fmaxf(m_run, mx);
            const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
            m_run = m_new;

            // Weights rounded to bf16 for the P*V product; the row sum uses
            // the same rounded weights, so O stays a convex combination of
            // the rows of V.
            bf16x8 pb[BN / 16];
            float psum = 0.f;
#pragma unroll
            for (int kb = 0; kb < BN / 32; ++kb) {
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const bf16 p = (bf16)__builtin_amdgcn_exp2f(sacc[kb][j] - m_use);
                    psum += (float)p;
                    pb[kb * 2 + (j >> 3)][j & 7] = p;
                }
            }
            l_run = l_run * alpha + psum;

#pragma unroll
            for (int db = 0; db < D / 32; ++db) {
#pragma unroll
                for (int j = 0; j < 16; ++j) oacc[db][j] *= alpha;
            }

            // O^T += V^T P^T.  Lane (feature d, half hi) supplies V for keys
            // 16ks + 4hi + {0..3} and 16ks + 8 + 4hi + {0..3}, the same keys
            // its P operand holds.
#pragma unroll
            for (int db = 0; db < D / 32; ++db) {
                const int d = db * 32 + l32;
                const int sw = vswz(d);
                const bf16* vrow = vt + d * BN;
#pragma unroll
                for (int ks2 = 0; ks2 < BN / 16; ++ks2) {
                    const int g1 = 4 * ks2 + hi;
                    const bf16x4 lo = *reinterpret_cast<const bf16x4*>(vrow + ((g1 ^ sw) * 4));
                    const bf16x4 hi4 = *reinterpret_cast<const bf16x4*>(vrow + (((g1 + 2) ^ sw) * 4));
                    const bf16x8 a = {lo[0], lo[1], lo[2], lo[3], hi4[0], hi4[1], hi4[2], hi4[3]};
                    oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[ks2], oacc[db], 0, 0, 0);
                }
            }
        }

        if (has_next) store_tile((t + 1) & 1);
        __syncthreads();
    }

    // Epilogue: O = O_acc / l, rounded once to bf16.  Rows past T_q fall
    // outside the buffer range and their stores are dropped.
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const float inv = 1.f / l_tot;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            bf16x4 w;
#pragma unroll
            for (int r = 0; r < 4; ++r) w[r] = (bf16)(oacc[db][4 * g4 + r] * inv);
            buf_store_b64(__builtin_bit_cast(u32x2, w), rO,
                          (uint32_t)(my_row * D + db * 32 + 8 * g4 + 4 * hi) * 2);
        }
    }
}

template <int D, int BN, bool CAUSAL>
hipError_t launch_one(const PrefillArgs& a, hipStream_t s) {
    const int n_qt = (a.T_q + kBM - 1) / kBM;
    const long long grid = (long long)a.B * a.H_q * n_qt;
    return launch_kernel(prefill_bf16_kernel<D, BN, CAUSAL>, dim3((unsigned)grid), dim3(kThreads), 0, s,
                         static_cast<const bf16*>(a.q), static_cast<const bf16*>(a.k),
                         static_cast<const bf16*>(a.v), static_cast<bf16*>(a.o), a.B, a.H_q, a.H_kv,
                         a.T_q, a.T_kv, n_qt, a.scale_log2);
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t s) {
    if (a.D == 128) {
        return a.causal ? launch_one<128, 64, true>(a, s) : launch_one<128, 64, false>(a, s);
    }
    return a.causal ? launch_one<64, 128, true>(a, s) : launch_one<64, 128, false>(a, s);
}

}  // namespace attn
