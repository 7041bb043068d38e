// bf16 attention forward for decode (one query token per sequence), gfx950.
//
// Decode is a vector against the whole KV cache and is bound by reading K
// and V from HBM (learn-cuda-from-scratch Ch. 11 "Attention", section
// 11.8.2; AIInfraGuide "3.3 Self-Attention机制深入理解", section 11.2).
// Two passes:
//
//   1. split pass: the keys of each (batch, kv head) are cut into
//      n_splits contiguous ranges.  One wave owns one range and all query
//      heads that read this kv head (up to 32 per wave), so K and V are read
//      from HBM once for the whole group (the GQA saving of section 11.8.1).
//      It keeps the online-softmax state (running max m in log2 units, sum
//      l, unnormalised output) and writes it to the workspace.
//   2. combine pass: per (batch, q head) the split states are merged with the
//      block-merge rule of AIInfraGuide section 12.3:
//      m = max m_s, l = sum l_s 2^(m_s - m), O = sum O_s 2^(m_s - m) / l.
//
// The split pass uses the same MFMA layout as the prefill kernel with the
// query heads of the group as the 32 MFMA columns: S^T = K Q^T on
// v_mfma_f32_32x32x16_bf16, then O^T += V^T P^T.  Each wave streams 32-key
// tiles of K and V with 16-byte loads that read whole rows, keeps the next
// tile in flight in registers, and stages the current one in its own LDS
// region (V transposed for the P*V operand).
#include "kernel_common.h"

namespace attn {
namespace {

constexpr int kWavesPerBlock = 4;
constexpr int kBN = 32;  // keys per tile

__device__ inline uint32_t pack_lo(uint32_t a, uint32_t b) { return (a & 0xffffu) | (b << 16); }
__device__ inline uint32_t pack_hi(uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xffff0000u); }

// Transposed-V swizzle for 32-key rows (8 groups of 4 keys): conflict-free
// reads, at most 2-way conflicts on the transposing writes.
__device__ inline int vswz8(int d) { return ((d >> 3) ^ (d >> 1)) & 7; }

template <int D>
__global__ __launch_bounds__(64 * kWavesPerBlock) void decode_split_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    float* __restrict__ ws_o, float* __restrict__ ws_ml, int H_q, int H_kv, int T_kv,
    int n_splits, int kps, int n_hb, int total_waves, float scale_log2) {
    constexpr int CPR = D / 8;
    constexpr int KSW = CPR - 1;
    constexpr int STAGE = 2 * kBN * D;
    constexpr int NK = kBN * CPR / 64;
    constexpr int NVQ = (kBN / 4) * CPR / 64;
    static_assert(NK * 64 == kBN * CPR && NVQ * 64 == (kBN / 4) * CPR, "tile split");

    __shared__ __attribute__((aligned(16))) bf16 smem[kWavesPerBlock * STAGE];

    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int l32 = lane & 31;
    const int hi = lane >> 5;
    const int gw = blockIdx.x * kWavesPerBlock + wave;
    if (gw >= total_waves) return;  // no block-wide barriers in this kernel

    const int split = gw % n_splits;
    const int rest = gw / n_splits;
    const int hb = rest % n_hb;
    const int unit = rest / n_hb;
    const int b = unit / H_kv;
    const int hk = unit - b * H_kv;
    const int G = H_q / H_kv;
    const int gi = hb * 32 + l32;
    const bool valid = gi < G;
    const int hq = hk * G + gi;

    const int k0 = split * kps;
    const int k1 = min(T_kv, k0 + kps);
    const int n_t = (k1 - k0 + kBN - 1) / kBN;

    // This split's keys only: loads past k1 read as zero.
    const uint32_t split_bytes = (uint32_t)(k1 - k0) * D * 2;
    const auto rK = make_rsrc(K + ((size_t)unit * T_kv + k0) * D, split_bytes);
    const auto rV = make_rsrc(V + ((size_t)unit * T_kv + k0) * D, split_bytes);
    // Query heads of this group: heads past the group read as zero.
    const int g_rows = min(32, G - hb * 32);
    const auto rQ = make_rsrc(Q + (size_t)(b * H_q + hk * G + hb * 32) * D, (uint32_t)g_rows * D * 2);

    bf16x8 qf[D / 16];
#pragma unroll
    for (int s = 0; s < D / 16; ++s)
        qf[s] = __builtin_bit_cast(bf16x8, buf_load_b128(rQ, (uint32_t)(l32 * D + 16 * s + 8 * hi) * 2));

    bf16* ks = smem + wave * STAGE;
    bf16* vt = ks + kBN * D;

    u32x4 kr[NK];
    u32x4 vr[NVQ][4];

    // jr: first key of the tile, relative to k0.
    auto load_tile = [&](int jr) {
#pragma unroll
        for (int i = 0; i < NK; ++i) {
            const int c = lane + i * 64;
            const int row = c / CPR, ch = c % CPR;
            kr[i] = buf_load_b128(rK, (uint32_t)((jr + row) * D + ch * 8) * 2);
        }
#pragma unroll
        for (int i = 0; i < NVQ; ++i) {
            const int u = lane + i * 64;
            const int ch = u % CPR, kq = u / CPR;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                vr[i][r] = buf_load_b128(rV, (uint32_t)((jr + 4 * kq + r) * D + ch * 8) * 2);
        }
    };

    auto store_tile = [&]() {
#pragma unroll
        for (int i = 0; i < NK; ++i) {
            const int c = lane + i * 64;
            const int row = c / CPR, ch = c % CPR;
            *reinterpret_cast<u32x4*>(ks + row * D + ((ch ^ (row & KSW)) * 8)) = kr[i];
        }
#pragma unroll
        for (int i = 0; i < NVQ; ++i) {
            const int u = lane + i * 64;
            const int ch = u % CPR, kq = u / CPR;
            const u32x4 w0 = vr[i][0], w1 = vr[i][1], w2 = vr[i][2], w3 = vr[i][3];
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const int d0 = ch * 8 + 2 * w;
                const int d1 = d0 + 1;
                const u32x2 lo = {pack_lo(w0[w], w1[w]), pack_lo(w2[w], w3[w])};
                const u32x2 hi2 = {pack_hi(w0[w], w1[w]), pack_hi(w2[w], w3[w])};
                *reinterpret_cast<u32x2*>(vt + d0 * kBN + ((kq ^ vswz8(d0)) * 4)) = lo;
                *reinterpret_cast<u32x2*>(vt + d1 * kBN + ((kq ^ vswz8(d1)) * 4)) = hi2;
            }
        }
    };

    f32x16 oacc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) oacc[db] = f32x16{};
    float m_run = -INFINITY;
    float l_run = 0.f;

    if (n_t > 0) load_tile(0);
    for (int t = 0; t < n_t; ++t) {
        const int j0 = k0 + t * kBN;
        // LDS operations of one wave complete in program order, so the
        // previous tile's reads are done before these writes land.
        store_tile();
        if (t + 1 < n_t) load_tile((t + 1) * kBN);

        f32x16 sacc = f32x16{};
        {
            const int key = l32;
            const bf16* krow = ks + key * D;
#pragma unroll
            for (int s = 0; s < D / 16; ++s) {
                const int ch = (2 * s + hi) ^ (key & KSW);
                const bf16x8 a = *reinterpret_cast<const bf16x8*>(krow + ch * 8);
                sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], sacc, 0, 0, 0);
            }
        }
        const bool need_mask = j0 + kBN > k1;
        float mx = -INFINITY;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            float x = sacc[j] * scale_log2;
            if (need_mask) {
                const int key = j0 + 8 * (j >> 2) + 4 * hi + (j & 3);
                x = key < k1 ? x : -INFINITY;
            }
            sacc[j] = x;
            mx = fmaxf(mx, x);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
        m_run = m_new;

        // bf16 weights for P*V; the row sum uses the same rounded weights.
        bf16x8 pb[2];
        float psum = 0.f;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const bf16 p = (bf16)__builtin_amdgcn_exp2f(sacc[j] - m_use);
            psum += (float)p;
            pb[j >> 3][j & 7] = p;
        }
        l_run = l_run * alpha + psum;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
#pragma unroll
            for (int j = 0; j < 16; ++j) oacc[db][j] *= alpha;
        }
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
            const int d = db * 32 + l32;
            const int sw = vswz8(d);
            const bf16* vrow = vt + d * kBN;
#pragma unroll
            for (int ks2 = 0; ks2 < 2; ++ks2) {
                const int g1 = 4 * ks2 + hi;
                const bf16x4 lo = *reinterpret_cast<const bf16x4*>(vrow + ((g1 ^ sw) * 4));
                const bf16x4 hi4 = *reinterpret_cast<const bf16x4*>(vrow + (((g1 + 2) ^ sw) * 4));
                const bf16x8 a = {lo[0], lo[1], lo[2], lo[3], hi4[0], hi4[1], hi4[2], hi4[3]};
                oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[ks2], oacc[db], 0, 0, 0);
            }
        }
    }

    const float l_tot = l_run + __shfl_xor(l_run, 32);
    if (valid) {
        const size_t idx = (size_t)(b * H_q + hq) * n_splits + split;
        float* op = ws_o + idx * D + 4 * hi;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const f32x4 w = {oacc[db][4 * g4], oacc[db][4 * g4 + 1], oacc[db][4 * g4 + 2],
                                 oacc[db][4 * g4 + 3]};
                *reinterpret_cast<f32x4*>(op + db * 32 + 8 * g4) = w;
            }
        }
        if (hi == 0) {
            ws_ml[2 * idx] = m_run;
            ws_ml[2 * idx + 1] = l_tot;
        }
    }
}

// One wave per (batch, q head): merge the split states and write O.
template <int D>
__global__ __launch_bounds__(64) void decode_combine_kernel(const float* __restrict__ ws_o,
                                                            const float* __restrict__ ws_ml,
                                                            bf16* __restrict__ O, int n_splits) {
    const size_t row = blockIdx.x;
    const int lane = threadIdx.x;
    const float* ml = ws_ml + row * n_splits * 2;
    float m = -INFINITY;
    for (int s = 0; s < n_splits; ++s) m = fmaxf(m, ml[2 * s]);
    float L = 0.f;
    float acc[D / 64];
#pragma unroll
    for (int r = 0; r < D / 64; ++r) acc[r] = 0.f;
    const float* op = ws_o + row * n_splits * D + lane;
    for (int s = 0; s < n_splits; ++s) {
        const float w = __builtin_amdgcn_exp2f(ml[2 * s] - m);
        L += ml[2 * s + 1] * w;
#pragma unroll
        for (int r = 0; r < D / 64; ++r) acc[r] += w * op[(size_t)s * D + 64 * r];
    }
    const float inv = 1.f / L;
#pragma unroll
    for (int r = 0; r < D / 64; ++r) O[row * D + lane + 64 * r] = (bf16)(acc[r] * inv);
}

template <int D>
hipError_t launch_d(const DecodeArgs& a, hipStream_t s) {
    const int G = a.H_q / a.H_kv;
    const int n_hb = (G + 31) / 32;
    const long long total_waves = (long long)a.B * a.H_kv * n_hb * a.n_splits;
    const long long blocks = (total_waves + kWavesPerBlock - 1) / kWavesPerBlock;
    hipError_t e = launch_kernel(decode_split_kernel<D>, dim3((unsigned)blocks), dim3(64 * kWavesPerBlock), 0, s,
                                 static_cast<const bf16*>(a.q), static_cast<const bf16*>(a.k),
                                 static_cast<const bf16*>(a.v), a.ws_o, a.ws_ml, a.H_q, a.H_kv, a.T_kv,
                                 a.n_splits, a.keys_per_split, n_hb, (int)total_waves, a.scale_log2);
    if (e != hipSuccess) return e;
    const long long rows = (long long)a.B * a.H_q;
    return launch_kernel(decode_combine_kernel<D>, dim3((unsigned)rows), dim3(64), 0, s,
                         static_cast<const float*>(a.ws_o), static_cast<const float*>(a.ws_ml),
                         static_cast<bf16*>(a.o), a.n_splits);
}

}  // namespace

hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t s) {
    return a.D == 128 ? launch_d<128>(a, s) : launch_d<64>(a, s);
}

}  // namespace attn
