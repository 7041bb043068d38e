// Fused QKV projection for gfx950: one bf16 GEMM Y = X W^T over the
// concatenated projection weights, with an epilogue that splits the output
// columns into Q, K and V and writes each in the head-major layout the
// attention kernels read.
//
// Method (learn-cuda-from-scratch Ch. 11 "Attention", section 11.2: Q, K and
// V are three linear maps of the same input X; section 11.8.1: the query
// heads and the (fewer) kv heads are column blocks of those maps):
//
//     Y[m, n] = sum_k X[m, k] W[n, k]          m = token, n = output feature
//     n <  H_q D            : Q[b, n / D,              t, n % D]
//     n <  (H_q + H_kv) D   : K[b, (n - H_q D) / D,    t, n % D]
//     otherwise             : V[b, (n - H_q D - H_kv D) / D, t, n % D]
//
// with m = b T + t.  W is stored [N][d_model] (one row per output feature,
// the layout of a linear layer's weight), so both GEMM operands are
// contiguous along the reduction dimension.
//
// gfx950 mapping:
//   * 8 waves per workgroup, workgroup tile 256 tokens x 256 features, wave
//     tile 64 tokens x 128 features.  Y^T = W X^T on
//     v_mfma_f32_32x32x16_bf16 (A = 32 features x 16 k of W, B = 32 tokens x
//     16 k of X): each lane's accumulator holds one token and 4-feature runs,
//     so the epilogue writes 8-byte runs of one output row.  Every W
//     fragment feeds 2 MFMAs and every X fragment 4 (0.75 KiB of LDS per
//     MFMA).
//   * 64-wide k tiles of X and W go HBM -> LDS with 16-byte buffer loads that
//     write LDS directly, double buffered; 128-byte rows use the same XOR
//     swizzle of 16-byte chunks as the attention kernels' K tiles (conflict-
//     free ds_read_b128 operand reads).  The fragments of the next k step
//     are read while the current step's MFMAs run, and the last k step's
//     MFMAs of each tile are issued after the next tile's barrier (their
//     fragments are already in registers), so they cover the barrier and
//     the first LDS round trip of the next tile; the 8 loads of the tile
//     after that go out between those MFMAs, one after each.
//   * Each XCD takes a compact block of output tiles (grouped tile order),
//     so the X and W tiles it reads are shared through its own L2.
//   * Tokens past B T and features past N read as zero (range-checked buffer
//     resources) and are not stored.  d_model must be a multiple of 64.
#include "launch.h"

namespace attn {
namespace {

// s_waitcnt lgkmcnt(N) that also redefines the six fragments g, so no use
// of them can be scheduled before it (LDS reads complete in issue order).
template <int N>
__device__ inline void lds_wait_bind6(bf16x8 (&g)[6]) {
    static_assert(N >= 0 && N <= 15, "lgkmcnt is 4 bits");
    asm volatile("s_waitcnt lgkmcnt(%6)"
                 : "+v"(g[0]), "+v"(g[1]), "+v"(g[2]), "+v"(g[3]), "+v"(g[4]), "+v"(g[5])
                 : "n"(N));
}

constexpr int kWaves = 8;
constexpr int kTM = 256;   // tokens per workgroup
constexpr int kTN = 256;   // features per workgroup
constexpr int kTK = 64;    // reduction elements per k tile
constexpr int kRowB = kTK * 2;                 // bytes per tile row (128)
constexpr int kCPR = kRowB / 16;               // 16-byte chunks per row (8)
constexpr int kXTile = kTM * kRowB;            // 32 KiB
constexpr int kWTile = kTN * kRowB;            // 32 KiB
constexpr int kStage = kXTile + kWTile;
constexpr int kGroupM = 8;  // token tiles per group of the tile order

template <int D>
__global__ __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(2, 2))) void
qkv_project_kernel(const bf16* __restrict__ X, const bf16* __restrict__ W, bf16* __restrict__ Qo,
                   bf16* __restrict__ Ko, bf16* __restrict__ Vo, int M, int N, int d_model, int T,
                   int H_q, int H_kv, int n_nt) {
    __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * kStage];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int hi = lane >> 5;
    const int wt = wave & 3;   // token block of 64
    const int wf = wave >> 2;  // feature block of 128

    // Workgroup id -> output tile.  Dispatch sends id to XCD (id mod 8).
    // Each XCD takes a contiguous range of tiles in grouped order (kGroupM
    // token tiles per group, feature tiles walking within the group), i.e.
    // a compact block of rows and columns, so the X and W tiles it reads
    // are shared through its own L2; the plain row-major order gave every
    // XCD every token tile.
    const int n_tiles = (int)gridDim.x;
    int v = (int)blockIdx.x;
    if ((n_tiles & 7) == 0) v = (v & 7) * (n_tiles >> 3) + (v >> 3);
    const int n_mt = n_tiles / n_nt;
    const int group = v / (kGroupM * n_nt);
    const int first_m = group * kGroupM;
    const int gsize = min(n_mt - first_m, kGroupM);
    const int in_group = v - group * kGroupM * n_nt;
    const int mt = first_m + in_group % gsize, nt = in_group / gsize;
    const int m0 = mt * kTM, n0 = nt * kTN;

    // The row counts are wave-uniform, but the clamp compiles to a vector
    // instruction; readfirstlane keeps the buffer resources in scalar
    // registers (otherwise every tile load is wrapped in a loop over
    // distinct resource values).
    const uint32_t rowb = (uint32_t)d_model * 2;
    const int x_rows = __builtin_amdgcn_readfirstlane(max(0, min(kTM, M - m0)));
    const int w_rows = __builtin_amdgcn_readfirstlane(max(0, min(kTN, N - n0)));
    const auto rX = make_rsrc(X + (size_t)m0 * d_model, (uint32_t)x_rows * rowb);
    const auto rW = make_rsrc(W + (size_t)n0 * d_model, (uint32_t)w_rows * rowb);

    // One k tile of X (256 rows) and of W (256 rows): 32 + 32 loads of
    // 1 KiB, 4 + 4 per wave.  LDS holds the X tiles of both stages, then
    // the W tiles of both stages, so every operand read's stage and block
    // offset fits the 16-bit immediate of ds_read_b128.
    // Load i (0 .. 2 NL - 1) of k tile kt alone: i < NL a piece of X, else of W.
    auto issue_one = [&](int kt, int buf, int i) {
        constexpr int NL = kXTile / (1024 * kWaves);
        const int n = i % NL;
        const int blk = wave * NL + n;
        const int p = blk * 64 + lane;
        const int row = p / kCPR;
        const int logical = (p % kCPR) ^ swz<kCPR>(row);
        const uint32_t off = (uint32_t)row * rowb + (uint32_t)kt * kRowB + logical * 16;
        if (i < NL) buf_load_lds16(rX, smem + buf * kXTile + blk * 1024, off);
        else buf_load_lds16(rW, smem + 2 * kXTile + buf * kWTile + blk * 1024, off);
    };
    auto issue = [&](int kt, int buf) {
        unsigned char* xs = smem + buf * kXTile;
        unsigned char* ws = smem + 2 * kXTile + buf * kWTile;
        const uint32_t kb = (uint32_t)kt * kRowB;
#pragma unroll
        for (int n = 0; n < kXTile / (1024 * kWaves); ++n) {
            const int blk = wave * (kXTile / (1024 * kWaves)) + n;
            const int p = blk * 64 + lane;
            const int row = p / kCPR;
            const int logical = (p % kCPR) ^ swz<kCPR>(row);
            buf_load_lds16(rX, xs + blk * 1024, (uint32_t)row * rowb + kb + logical * 16);
            buf_load_lds16(rW, ws + blk * 1024, (uint32_t)row * rowb + kb + logical * 16);
        }
    };

    f32x16 acc[4][2];
#pragma unroll
    for (int fb = 0; fb < 4; ++fb) {
        acc[fb][0] = f32x16{};
        acc[fb][1] = f32x16{};
    }

    const int n_kt = d_model / kTK;
    issue(0, 0);
    // Operand fragments: lane (row l32 of a 32-row block, half hi) reads
    // the 16-byte chunk 2s + hi of its row for k step s, stored at chunk
    // (2s + hi) ^ swz(row).  swz depends on the row's low 4 bits only, so
    // every block of the wave shares the lane's chunk, and step s flips
    // bits 5-6 of the step-0 address: address = a0 ^ 32s, plus immediates
    // for the stage and the 32-row block.
    const uint32_t c0 = (uint32_t)((hi ^ swz<kCPR>(l32)) * 16);
    const uint32_t xa0 = lds_u32(smem) + (uint32_t)((wt * 64 + l32) * kRowB) + c0;
    const uint32_t wa0 = lds_u32(smem) + 2 * kXTile + (uint32_t)((wf * 128 + l32) * kRowB) + c0;
    uint32_t xa[kTK / 16], wa[kTK / 16];
#pragma unroll
    for (int st = 0; st < kTK / 16; ++st) {
        xa[st] = xa0 ^ (uint32_t)(32 * st);
        wa[st] = wa0 ^ (uint32_t)(32 * st);
    }
    // The fragments of k step s + 1 are read (inline assembly, waits bound
    // to the fragment registers) while the 8 MFMAs of step s run; the
    // compiler's own reads were issued only a few MFMAs ahead.
    // Fragments of the previous tile's last k step: multiplied after the
    // barrier, while the first reads of the next tile are in flight (the
    // accumulation order of every output is unchanged).
    bf16x8 g[6];
    auto tile = [&](int kt, auto stage) {
        constexpr int B = decltype(stage)::value;
        wait_vmem_all();
        __syncthreads();  // tile kt landed for every wave; the other stage is free
        bf16x8 f[2][6];  // [ring slot][X block 0, 1, W block 0..3]
        auto read = [&](bf16x8 (&r)[6], auto step) {
            constexpr int S = decltype(step)::value;
            r[0] = ds_read_b128_asm<B * kXTile>(xa[S]);
            r[1] = ds_read_b128_asm<B * kXTile + 32 * kRowB>(xa[S]);
            r[2] = ds_read_b128_asm<B * kWTile>(wa[S]);
            r[3] = ds_read_b128_asm<B * kWTile + 32 * kRowB>(wa[S]);
            r[4] = ds_read_b128_asm<B * kWTile + 64 * kRowB>(wa[S]);
            r[5] = ds_read_b128_asm<B * kWTile + 96 * kRowB>(wa[S]);
        };
        auto mma = [&](bf16x8 (&r)[6]) {
#pragma unroll
            for (int fb = 0; fb < 4; ++fb) {
#pragma unroll
                for (int tb = 0; tb < 2; ++tb)
                    acc[fb][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(r[2 + fb], r[tb], acc[fb][tb], 0, 0, 0);
            }
        };
        read(f[0], std::integral_constant<int, 0>{});
        // The previous tile's last step with tile kt + 1's loads between its
        // MFMAs, one after each (+2.9% over issuing the 8 loads together
        // right after the barrier).
        const bool more = kt + 1 < n_kt;
        if (kt > 0) {
#pragma unroll
            for (int fb = 0; fb < 4; ++fb) {
#pragma unroll
                for (int tb = 0; tb < 2; ++tb) {
                    acc[fb][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(g[2 + fb], g[tb], acc[fb][tb], 0, 0, 0);
                    if (more) issue_one(kt + 1, B ^ 1, fb * 2 + tb);
                }
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
                __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // one vector-memory read
            }
        } else if (more) {
            issue(kt + 1, B ^ 1);
        }
        read(f[1], std::integral_constant<int, 1>{});
        lds_wait_bind6<6>(f[0]);
        mma(f[0]);
        read(f[0], std::integral_constant<int, 2>{});
        lds_wait_bind6<6>(f[1]);
        mma(f[1]);
        read(g, std::integral_constant<int, 3>{});
        lds_wait_bind6<6>(f[0]);
        mma(f[0]);
        lds_wait_bind6<0>(g);  // before the next barrier: stage B is refilled after it
    };
    for (int kt = 0; kt < n_kt; kt += 2) {
        tile(kt, std::integral_constant<int, 0>{});
        if (kt + 1 < n_kt) tile(kt + 1, std::integral_constant<int, 1>{});
    }
#pragma unroll
    for (int fb = 0; fb < 4; ++fb) {
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
            acc[fb][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(g[2 + fb], g[tb], acc[fb][tb], 0, 0, 0);
    }

    // Epilogue: lane (token column l32, half hi) holds features
    // 8 (j / 4) + 4 hi + j % 4 of each 32-feature block: runs of 4 features
    // of one token, stored as 8 bytes.  A 32-feature block never straddles
    // a head (D is 64 or 128).
    const int qn = H_q * D, kn = H_kv * D;
    const uint32_t q_bytes = (uint32_t)((size_t)M * qn * 2), kv_bytes = (uint32_t)((size_t)M * kn * 2);
    const auto rQ = make_rsrc(Qo, q_bytes);
    const auto rK = make_rsrc(Ko, kv_bytes);
    const auto rV = make_rsrc(Vo, kv_bytes);
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
        const int m = m0 + wt * 64 + tb * 32 + l32;
        const int b = m / T, t = m - b * T;
        const bool m_ok = m < M;
#pragma unroll
        for (int fb = 0; fb < 4; ++fb) {
            const int nb = n0 + wf * 128 + fb * 32;  // first feature of the block (uniform)
            if (nb >= N) continue;
            int col, H;
            __amdgpu_buffer_rsrc_t r = rQ;
            if (nb < qn) {
                col = nb;
                H = H_q;
            } else if (nb < qn + kn) {
                col = nb - qn;
                H = H_kv;
                r = rK;
            } else {
                col = nb - qn - kn;
                H = H_kv;
                r = rV;
            }
            const int h = col / D, d0 = col - h * D;
            const uint32_t base = (uint32_t)(((size_t)(b * H + h) * T + t) * D + d0) * 2;
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                bf16x4 w;
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) w[r4] = (bf16)acc[fb][tb][4 * g4 + r4];
                const uint32_t off = m_ok ? base + (uint32_t)(8 * g4 + 4 * hi) * 2 : 0xFFFFFFF0u;
                buf_store_b64(__builtin_bit_cast(u32x2, w), r, off);
            }
        }
    }
}

template <int D>
hipError_t launch_q(const QkvArgs& a, hipStream_t s) {
    const int n_mt = (a.M + kTM - 1) / kTM;
    const int n_nt = (a.N + kTN - 1) / kTN;
    return launch_kernel(qkv_project_kernel<D>, dim3((unsigned)((long long)n_mt * n_nt)),
                         dim3(64 * kWaves), 0, s, static_cast<const bf16*>(a.x),
                         static_cast<const bf16*>(a.w), static_cast<bf16*>(a.q),
                         static_cast<bf16*>(a.k), static_cast<bf16*>(a.v), a.M, a.N, a.d_model, a.T,
                         a.H_q, a.H_kv, n_nt);
}

}  // namespace

hipError_t launch_qkv_bf16(const QkvArgs& a, hipStream_t s) {
    return a.D == 128 ? launch_q<128>(a, s) : launch_q<64>(a, s);
}

}  // namespace attn
