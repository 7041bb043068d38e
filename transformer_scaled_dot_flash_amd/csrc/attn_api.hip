// C ABI of the attention forward: argument checks and dispatch.
// Every check runs on the host before any HIP call, so all error paths can
// be exercised without a GPU.  The contract is documented in include/attn.h.
#include <float.h>
#include <math.h>

#include <mutex>

#include "attn.h"
#include "launch.h"

namespace {

thread_local int g_last_hip_error = 0;

constexpr int kMaxSplits = 1024;
constexpr int kDecodeBlock = 32;  // keys per decode tile; splits are multiples of it

size_t elem_size(int dtype) { return dtype == ATTN_F32 ? 4 : 2; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return na && nb && a0 < b0 + nb && b0 < a0 + na;
}

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

// Shape / parameter checks shared by both entry points.
attn_status_t check_params(int B, int H_q, int H_kv, int T_q, int T_kv, int D, int dtype,
                           float scale) {
    if (B < 0 || T_q < 0 || H_q <= 0 || H_kv <= 0 || T_kv <= 0) return ATTN_ERR_INVALID_SHAPE;
    if (H_q % H_kv != 0) return ATTN_ERR_INVALID_SHAPE;
    if (dtype != ATTN_F32 && dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
    if (D != 64 && D != 128) return ATTN_ERR_UNSUPPORTED;
    if (!isfinite(scale)) return ATTN_ERR_INVALID_SCALE;
    // One (batch, head) slice of any tensor must stay below 2 GiB: kernels
    // address it with 32-bit offsets.
    const long long es = (long long)elem_size(dtype);
    if ((long long)T_q * D * es >= (1LL << 31) || (long long)T_kv * D * es >= (1LL << 31))
        return ATTN_ERR_INVALID_SHAPE;
    return ATTN_OK;
}

attn_status_t check_tensors(const void* q, const void* k, const void* v, const void* o, int B,
                            int H_q, int H_kv, int T_q, int T_kv, int D, int dtype) {
    if (!q || !k || !v || !o) return ATTN_ERR_NULL_PTR;
    if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(o)) return ATTN_ERR_ALIGNMENT;
    const size_t es = elem_size(dtype);
    const size_t nq = (size_t)B * H_q * T_q * D * es;
    const size_t nkv = (size_t)B * H_kv * T_kv * D * es;
    if (overlaps(o, nq, q, nq) || overlaps(o, nq, k, nkv) || overlaps(o, nq, v, nkv))
        return ATTN_ERR_ALIAS;
    return ATTN_OK;
}

attn_status_t hip_status(hipError_t e) {
    if (e == hipSuccess) return ATTN_OK;
    g_last_hip_error = (int)e;
    return ATTN_ERR_HIP;
}

float log2_scale(float scale) { return (float)((double)scale * attn::kLog2e); }

// The bf16 kernels take a positive multiplier: a negative scale is applied
// by negating Q (exact), and a zero scale by the smallest normal float, which
// gives bitwise the same weights (every exponent rounds to 2^0).
void positive_scale(float scale, float* c, int* neg) {
    double v = (double)scale * attn::kLog2e;
    *neg = v < 0 ? 1 : 0;
    v = v < 0 ? -v : v;
    float f = (float)v;
    if (!(f >= FLT_MIN)) f = FLT_MIN;
    *c = f;
}

struct SplitPlan {
    int n_splits;
    int keys_per_split;
};

int default_splits(int B, int H_q, int H_kv, int T_kv, int D) {
    const int G = H_q / H_kv;
    const long long groups = (long long)B * H_kv * ((G + 31) / 32);
    const int n_blocks = (T_kv + kDecodeBlock - 1) / kDecodeBlock;
    // One wave per (group, split).  The cache streams fastest with one full
    // round of waves: 768 at D = 128 (three per CU), 1024 at D = 64 (four);
    // measured over split counts 1..128 on eleven shapes, 512 waves ran 3-6%
    // (D = 128) and up to a third (D = 64) slower, and a partial second round
    // (e.g. 1024 waves at D = 128) 15-20% slower.  So: as many splits as fit
    // in one round (at least one; enough groups -> one split and no combine
    // pass), keeping >= 4 tiles per split.
    const long long target = D == 64 ? 1024 : 768;
    long long want = target / groups;
    long long cap = n_blocks / 4;
    if (cap < 1) cap = 1;
    if (want > cap) want = cap;
    if (want > kMaxSplits) want = kMaxSplits;
    if (want < 1) want = 1;
    return (int)want;
}

SplitPlan plan_splits(int B, int H_q, int H_kv, int T_kv, int D, int requested) {
    const int n_blocks = (T_kv + kDecodeBlock - 1) / kDecodeBlock;
    int n = requested > 0 ? requested : default_splits(B, H_q, H_kv, T_kv, D);
    if (n > n_blocks) n = n_blocks;
    const int blocks_per = (n_blocks + n - 1) / n;
    SplitPlan p;
    p.keys_per_split = blocks_per * kDecodeBlock;
    p.n_splits = (T_kv + p.keys_per_split - 1) / p.keys_per_split;  // no empty split
    return p;
}

// Workspace of a split plan: partial outputs [B][H_q][S][D] fp32, then
// (max, sum) [B][H_q][S][2] fp32.
size_t decode_ws_bytes(int B, int H_q, int D, const SplitPlan& p) {
    if (p.n_splits == 1) return 0;  // the split pass writes O directly
    return (size_t)B * H_q * p.n_splits * (D + 2) * sizeof(float);
}

// Paged cache: page_size a power of two in [16, 65536]; returns log2 or -1.
int page_shift_of(int page_size) {
    if (page_size < 16 || page_size > 65536 || (page_size & (page_size - 1))) return -1;
    int s = 0;
    while ((1 << s) < page_size) ++s;
    return s;
}

attn_status_t check_paged_params(int B, int H_q, int H_kv, int D, int page_size, int num_pages,
                                 int max_pages, int dtype, float scale, int num_splits) {
    if (B < 0 || H_q <= 0 || H_kv <= 0 || num_pages <= 0 || max_pages <= 0) return ATTN_ERR_INVALID_SHAPE;
    if (H_q % H_kv != 0) return ATTN_ERR_INVALID_SHAPE;
    if (dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
    if (D != 64 && D != 128) return ATTN_ERR_UNSUPPORTED;
    if (page_shift_of(page_size) < 0) return ATTN_ERR_UNSUPPORTED;
    if (num_splits < 0 || num_splits > kMaxSplits) return ATTN_ERR_UNSUPPORTED;
    if (!isfinite(scale)) return ATTN_ERR_INVALID_SCALE;
    // Key positions are 32-bit and one page of one kv head is addressed with
    // 32-bit offsets.
    if ((long long)max_pages * page_size > (1LL << 30)) return ATTN_ERR_INVALID_SHAPE;
    const long long waves = (long long)B * H_kv * ((H_q / H_kv + 31) / 32) * kMaxSplits;
    if (waves / 4 > 0x7fffffffLL || (long long)B * H_q > 0x7fffffffLL) return ATTN_ERR_INVALID_SHAPE;
    return ATTN_OK;
}

// Workspace pointers of a decode launch (partial outputs, then (max, sum)).
void set_workspace(attn::DecodeArgs& a, void* ws, int B, int H_q, int D, const SplitPlan& p) {
    a.ws_o = static_cast<float*>(ws);
    a.ws_ml = ws ? a.ws_o + (size_t)B * H_q * p.n_splits * D : nullptr;
}

// The bf16 decode launch shared by attn_fwd_decode and
// attn_fwd_decode_noalloc: `ws` holds the split partials (unused with one
// split).
attn_status_t decode_bf16(const void* q, const void* k, const void* v, void* o, int B, int H_q,
                          int H_kv, int T_kv, int D, float scale, const SplitPlan& p, void* ws,
                          hipStream_t s) {
    attn::DecodeArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.B = B;
    a.H_q = H_q;
    a.H_kv = H_kv;
    a.T_kv = T_kv;
    a.D = D;
    positive_scale(scale, &a.c_log2, &a.neg_q);
    a.n_splits = p.n_splits;
    a.keys_per_split = p.keys_per_split;
    set_workspace(a, ws, B, H_q, D, p);
    return hip_status(attn::launch_decode_bf16(a, s));
}

// fp32 decode: the fp32 forward with one query row (no workspace).
attn_status_t decode_f32(const void* q, const void* k, const void* v, void* o, int B, int H_q,
                         int H_kv, int T_kv, int D, float scale, hipStream_t s) {
    attn::PrefillArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.B = B;
    a.H_q = H_q;
    a.H_kv = H_kv;
    a.T_q = 1;
    a.T_kv = T_kv;
    a.D = D;
    a.causal = 0;
    a.scale = scale;
    a.scale_log2 = log2_scale(scale);
    positive_scale(scale, &a.c_log2, &a.neg_q);
    return hip_status(attn::launch_prefill_f32(a, s));
}

// Checks every decode entry point shares (before any pointer is looked at).
attn_status_t check_decode_params(int B, int H_q, int H_kv, int T_q, int T_kv, int D, int dtype,
                                  float scale, int num_splits) {
    attn_status_t st = check_params(B, H_q, H_kv, T_q, T_kv, D, dtype, scale);
    if (st != ATTN_OK) return st;
    if (T_q != 1) return ATTN_ERR_UNSUPPORTED;
    if (num_splits < 0 || num_splits > kMaxSplits) return ATTN_ERR_UNSUPPORTED;
    const long long waves = (long long)B * H_kv * ((H_q / H_kv + 31) / 32) * kMaxSplits;
    if (waves / 4 > 0x7fffffffLL || (long long)B * H_q > 0x7fffffffLL) return ATTN_ERR_INVALID_SHAPE;
    return ATTN_OK;
}

// Scratch of the no-allocation decode: the split partials of one call live
// here instead of in a caller's workspace.  Each GPU the library runs on
// holds its own copy from the module's load until the process ends.  In host
// code `scratch` names a host-side stand-in, not device memory: only the
// address returned by hipGetSymbolAddress (one per device) is passed to
// kernels.
static __device__ __align__(256) unsigned char scratch[ATTN_DECODE_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices];  // device address of `scratch` on each device (nullptr: not looked up)

// Device address of `scratch` on the device `s` launches on, looked up once
// per device with that device current.
attn_status_t scratch_for_stream(hipStream_t s, void** out) {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return hip_status(e);
    int dev = cur;
    if (s != nullptr) {
        hipDevice_t d = -1;
        e = hipStreamGetDevice(s, &d);
        if (e != hipSuccess) return hip_status(e);
        dev = (int)d;
    }
    if (dev < 0 || dev >= kMaxDevices) return hip_status(hipErrorInvalidDevice);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_dev[dev] == nullptr) {
        if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return hip_status(e);
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        const hipError_t e_back = (dev != cur) ? hipSetDevice(cur) : hipSuccess;
        if (e != hipSuccess) return hip_status(e);
        if (e_back != hipSuccess) return hip_status(e_back);
        if (p == nullptr) return hip_status(hipErrorInvalidSymbol);
        g_scratch_dev[dev] = p;
    }
    *out = g_scratch_dev[dev];
    return ATTN_OK;
}

}  // namespace

extern "C" {

attn_status_t attn_fwd_prefill(const void* q, const void* k, const void* v, void* o, int B,
                               int H_q, int H_kv, int T_q, int T_kv, int D, int causal,
                               float scale, int dtype, void* stream) {
    attn_status_t st = check_params(B, H_q, H_kv, T_q, T_kv, D, dtype, scale);
    if (st != ATTN_OK) return st;
    if (causal && T_q > T_kv) return ATTN_ERR_INVALID_SHAPE;
    // Grid limits: bf16 launches B*H_q*ceil(T_q/128) workgroups, fp32
    // B*H_kv*ceil(G*T_q/64); both must fit a 32-bit grid dimension.
    const long long G = H_q / H_kv;
    const long long g_bf16 = (long long)B * H_q * ((T_q + 127) / 128);
    const long long g_f32 = (long long)B * H_kv * ((G * T_q + 63) / 64);
    if (g_bf16 > 0x7fffffffLL || g_f32 > 0x7fffffffLL) return ATTN_ERR_INVALID_SHAPE;
    if (B == 0 || T_q == 0) return ATTN_OK;  // empty problem
    st = check_tensors(q, k, v, o, B, H_q, H_kv, T_q, T_kv, D, dtype);
    if (st != ATTN_OK) return st;

    attn::PrefillArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.B = B;
    a.H_q = H_q;
    a.H_kv = H_kv;
    a.T_q = T_q;
    a.T_kv = T_kv;
    a.D = D;
    a.causal = causal ? 1 : 0;
    a.scale = scale;
    a.scale_log2 = log2_scale(scale);
    positive_scale(scale, &a.c_log2, &a.neg_q);
    hipStream_t s = static_cast<hipStream_t>(stream);
    return hip_status(dtype == ATTN_BF16 ? attn::launch_prefill_bf16(a, s)
                                         : attn::launch_prefill_f32(a, s));
}

attn_status_t attn_fwd_prefill_window(const void* q, const void* k, const void* v, void* o, int B,
                                      int H_q, int H_kv, int T_q, int T_kv, int D, int window,
                                      float scale, int dtype, void* stream) {
    attn_status_t st = check_params(B, H_q, H_kv, T_q, T_kv, D, dtype, scale);
    if (st != ATTN_OK) return st;
    if (T_q > T_kv) return ATTN_ERR_INVALID_SHAPE;
    if (dtype != ATTN_BF16 || window < 1) return ATTN_ERR_UNSUPPORTED;
    const long long g_bf16 = (long long)B * H_q * ((T_q + 127) / 128);
    if (g_bf16 > 0x7fffffffLL) return ATTN_ERR_INVALID_SHAPE;
    if (B == 0 || T_q == 0) return ATTN_OK;
    st = check_tensors(q, k, v, o, B, H_q, H_kv, T_q, T_kv, D, dtype);
    if (st != ATTN_OK) return st;

    attn::PrefillArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.B = B;
    a.H_q = H_q;
    a.H_kv = H_kv;
    a.T_q = T_q;
    a.T_kv = T_kv;
    a.D = D;
    a.causal = 1;
    a.scale = scale;
    a.scale_log2 = log2_scale(scale);
    positive_scale(scale, &a.c_log2, &a.neg_q);
    a.window = window >= T_kv ? 0 : window;  // a window covering every key is plain causal
    return hip_status(attn::launch_prefill_bf16(a, static_cast<hipStream_t>(stream)));
}

attn_status_t attn_fwd_prefill_varlen(const void* q, const void* k, const void* v, void* o,
                                      const int* cu_seqlens_q, const int* cu_seqlens_k, int B,
                                      int H_q, int H_kv, int D, int total_q, int total_k,
                                      int max_seqlen_q, int max_seqlen_k, int causal, int window,
                                      float scale, int dtype, void* stream) {
    if (B < 0 || H_q <= 0 || H_kv <= 0 || total_q < 0 || total_k < 0 || max_seqlen_q < 0 ||
        max_seqlen_k < 0)
        return ATTN_ERR_INVALID_SHAPE;
    if (H_q % H_kv != 0) return ATTN_ERR_INVALID_SHAPE;
    if (dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
    if (D != 64 && D != 128) return ATTN_ERR_UNSUPPORTED;
    if (window < 0 || (window > 0 && !causal)) return ATTN_ERR_UNSUPPORTED;
    if (!isfinite(scale)) return ATTN_ERR_INVALID_SCALE;
    // Rows of one sequence are addressed with 32-bit byte offsets (with
    // margin for the last partial tile); the grid covers max_seqlen_q rows.
    if ((long long)(max_seqlen_q + 256) * H_q * D * 2 >= (1LL << 31) ||
        (long long)(max_seqlen_k + 64) * H_kv * D * 2 >= (1LL << 31))
        return ATTN_ERR_INVALID_SHAPE;
    if ((long long)B * H_q * ((max_seqlen_q + 127) / 128) > 0x7fffffffLL) return ATTN_ERR_INVALID_SHAPE;
    if (B == 0 || max_seqlen_q == 0 || total_q == 0) return ATTN_OK;
    if (!q || !k || !v || !o || !cu_seqlens_q || !cu_seqlens_k) return ATTN_ERR_NULL_PTR;
    if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(o) ||
        (reinterpret_cast<uintptr_t>(cu_seqlens_q) & 3u) || (reinterpret_cast<uintptr_t>(cu_seqlens_k) & 3u))
        return ATTN_ERR_ALIGNMENT;
    const size_t nq = (size_t)total_q * H_q * D * 2;
    const size_t nkv = (size_t)total_k * H_kv * D * 2;
    const size_t ncu = (size_t)(B + 1) * 4;
    if (overlaps(o, nq, q, nq) || overlaps(o, nq, k, nkv) || overlaps(o, nq, v, nkv) ||
        overlaps(o, nq, cu_seqlens_q, ncu) || overlaps(o, nq, cu_seqlens_k, ncu))
        return ATTN_ERR_ALIAS;

    attn::PrefillArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.B = B;
    a.H_q = H_q;
    a.H_kv = H_kv;
    a.T_q = max_seqlen_q;   // sizes the grid; each workgroup reads its sequence's lengths
    a.T_kv = max_seqlen_k;
    a.D = D;
    a.causal = causal ? 1 : 0;
    a.scale = scale;
    a.scale_log2 = log2_scale(scale);
    positive_scale(scale, &a.c_log2, &a.neg_q);
    a.window = window;
    a.cu_q = cu_seqlens_q;
    a.cu_k = cu_seqlens_k;
    a.total_q = total_q;
    return hip_status(attn::launch_prefill_bf16(a, static_cast<hipStream_t>(stream)));
}

attn_status_t attn_fwd_decode(const void* q, const void* k, const void* v, void* o, int B,
                              int H_q, int H_kv, int T_q, int T_kv, int D, int causal,
                              float scale, int dtype, int num_splits, void* workspace,
                              size_t workspace_bytes, void* stream) {
    attn_status_t st = check_decode_params(B, H_q, H_kv, T_q, T_kv, D, dtype, scale, num_splits);
    if (st != ATTN_OK) return st;
    (void)causal;  // one query row at the end of the keys sees every key
    if (B == 0) return ATTN_OK;
    st = check_tensors(q, k, v, o, B, H_q, H_kv, 1, T_kv, D, dtype);
    if (st != ATTN_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (dtype == ATTN_F32) return decode_f32(q, k, v, o, B, H_q, H_kv, T_kv, D, scale, s);

    const SplitPlan p = plan_splits(B, H_q, H_kv, T_kv, D, num_splits);
    const size_t need = decode_ws_bytes(B, H_q, D, p);
    if (need > 0 && (!workspace || workspace_bytes < need)) return ATTN_ERR_WORKSPACE;
    if (need > 0 && misaligned(workspace)) return ATTN_ERR_ALIGNMENT;
    const size_t es = elem_size(dtype);
    const size_t nq = (size_t)B * H_q * D * es;
    const size_t nkv = (size_t)B * H_kv * T_kv * D * es;
    if (overlaps(workspace, need, o, nq) || overlaps(workspace, need, q, nq) ||
        overlaps(workspace, need, k, nkv) || overlaps(workspace, need, v, nkv))
        return ATTN_ERR_ALIAS;
    return decode_bf16(q, k, v, o, B, H_q, H_kv, T_kv, D, scale, p, workspace, s);
}

attn_status_t attn_fwd_decode_noalloc(const void* q, const void* k, const void* v, void* o, int B,
                                      int H_q, int H_kv, int T_q, int T_kv, int D, int causal,
                                      float scale, int dtype, int num_splits, void* stream) {
    attn_status_t st = check_decode_params(B, H_q, H_kv, T_q, T_kv, D, dtype, scale, num_splits);
    if (st != ATTN_OK) return st;
    (void)causal;
    if (B == 0) return ATTN_OK;
    st = check_tensors(q, k, v, o, B, H_q, H_kv, 1, T_kv, D, dtype);
    if (st != ATTN_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (dtype == ATTN_F32) return decode_f32(q, k, v, o, B, H_q, H_kv, T_kv, D, scale, s);

    const SplitPlan p = plan_splits(B, H_q, H_kv, T_kv, D, num_splits);
    const size_t need = decode_ws_bytes(B, H_q, D, p);
    if (need > (size_t)ATTN_DECODE_SCRATCH_BYTES) return ATTN_ERR_SCRATCH;
    void* ws = nullptr;
    if (need > 0) {
        // The split pass overwrites every partial it hands to the combine
        // pass, so nothing in the scratch has to start at zero.
        st = scratch_for_stream(s, &ws);
        if (st != ATTN_OK) return st;
    }
    return decode_bf16(q, k, v, o, B, H_q, H_kv, T_kv, D, scale, p, ws, s);
}

size_t attn_fwd_decode_workspace_bytes(int B, int H_q, int H_kv, int T_kv, int D, int dtype,
                                       int num_splits) {
    if (check_params(B, H_q, H_kv, 1, T_kv, D, dtype, 1.0f) != ATTN_OK) return 0;
    if (num_splits < 0 || num_splits > kMaxSplits) return 0;
    if (dtype == ATTN_F32) return 0;
    return decode_ws_bytes(B, H_q, D, plan_splits(B, H_q, H_kv, T_kv, D, num_splits));
}

int attn_fwd_decode_default_splits(int B, int H_q, int H_kv, int T_kv, int D) {
    if (check_params(B, H_q, H_kv, 1, T_kv, D, ATTN_BF16, 1.0f) != ATTN_OK) return 0;
    return plan_splits(B, H_q, H_kv, T_kv, D, 0).n_splits;
}

attn_status_t attn_fwd_decode_paged(const void* q, const void* k_pages, const void* v_pages,
                                    void* o, const int* block_table, const int* seq_lens, int B,
                                    int H_q, int H_kv, int D, int page_size, int num_pages,
                                    int max_pages, float scale, int dtype, int num_splits,
                                    void* workspace, size_t workspace_bytes, void* stream) {
    attn_status_t st = check_paged_params(B, H_q, H_kv, D, page_size, num_pages, max_pages, dtype,
                                          scale, num_splits);
    if (st != ATTN_OK) return st;
    if (B == 0) return ATTN_OK;
    if (!q || !k_pages || !v_pages || !o || !block_table || !seq_lens) return ATTN_ERR_NULL_PTR;
    if (misaligned(q) || misaligned(k_pages) || misaligned(v_pages) || misaligned(o) ||
        (reinterpret_cast<uintptr_t>(block_table) & 3u) || (reinterpret_cast<uintptr_t>(seq_lens) & 3u))
        return ATTN_ERR_ALIGNMENT;
    const int T_max = max_pages * page_size;
    const SplitPlan p = plan_splits(B, H_q, H_kv, T_max, D, num_splits);
    const size_t need = decode_ws_bytes(B, H_q, D, p);
    if (need > 0 && (!workspace || workspace_bytes < need)) return ATTN_ERR_WORKSPACE;
    if (need > 0 && misaligned(workspace)) return ATTN_ERR_ALIGNMENT;
    const size_t nq = (size_t)B * H_q * D * 2;
    const size_t npool = (size_t)num_pages * H_kv * page_size * D * 2;
    const size_t nbt = (size_t)B * max_pages * 4, nsl = (size_t)B * 4;
    const void* ins[] = {q, k_pages, v_pages, block_table, seq_lens};
    const size_t lens[] = {nq, npool, npool, nbt, nsl};
    for (int i = 0; i < 5; ++i)
        if (overlaps(o, nq, ins[i], lens[i]) || overlaps(workspace, need, ins[i], lens[i]))
            return ATTN_ERR_ALIAS;
    if (overlaps(workspace, need, o, nq)) return ATTN_ERR_ALIAS;

    attn::DecodeArgs a{};
    a.q = q;
    a.k = k_pages;
    a.v = v_pages;
    a.o = o;
    a.B = B;
    a.H_q = H_q;
    a.H_kv = H_kv;
    a.T_kv = T_max;
    a.D = D;
    positive_scale(scale, &a.c_log2, &a.neg_q);
    a.n_splits = p.n_splits;
    a.keys_per_split = p.keys_per_split;
    set_workspace(a, need > 0 ? workspace : nullptr, B, H_q, D, p);
    a.paged.block_table = block_table;
    a.paged.seq_lens = seq_lens;
    a.paged.max_pages = max_pages;
    a.paged.page_shift = page_shift_of(page_size);
    a.paged.num_pages = num_pages;
    return hip_status(attn::launch_decode_bf16(a, static_cast<hipStream_t>(stream)));
}

size_t attn_fwd_decode_paged_workspace_bytes(int B, int H_q, int H_kv, int D, int page_size,
                                             int max_pages, int num_splits) {
    if (check_paged_params(B, H_q, H_kv, D, page_size, 1, max_pages, ATTN_BF16, 1.0f, num_splits) !=
        ATTN_OK)
        return 0;
    return decode_ws_bytes(B, H_q, D, plan_splits(B, H_q, H_kv, max_pages * page_size, D, num_splits));
}

attn_status_t attn_qkv_project(const void* x, const void* w, void* q, void* k, void* v, int B,
                               int T, int d_model, int H_q, int H_kv, int D, int dtype, void* stream) {
    if (B < 0 || T < 0 || d_model <= 0 || H_q <= 0 || H_kv <= 0) return ATTN_ERR_INVALID_SHAPE;
    if (H_q % H_kv != 0) return ATTN_ERR_INVALID_SHAPE;
    if (dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
    if (D != 64 && D != 128) return ATTN_ERR_UNSUPPORTED;
    if (d_model % 64 != 0) return ATTN_ERR_UNSUPPORTED;
    const long long M = (long long)B * T, N = (long long)(H_q + 2 * H_kv) * D;
    // every tensor is addressed with 32-bit byte offsets
    if (M * d_model * 2 >= (1LL << 31) || N * d_model * 2 >= (1LL << 31) ||
        M * H_q * D * 2 >= (1LL << 31) || (long long)d_model * 2 * 256 >= (1LL << 31))
        return ATTN_ERR_INVALID_SHAPE;
    if (M == 0) return ATTN_OK;
    if (!x || !w || !q || !k || !v) return ATTN_ERR_NULL_PTR;
    if (misaligned(x) || misaligned(w) || misaligned(q) || misaligned(k) || misaligned(v))
        return ATTN_ERR_ALIGNMENT;
    const size_t nx = (size_t)M * d_model * 2, nw = (size_t)N * d_model * 2;
    const size_t nq = (size_t)M * H_q * D * 2, nkv = (size_t)M * H_kv * D * 2;
    const void* outs[] = {q, k, v};
    const size_t olen[] = {nq, nkv, nkv};
    for (int i = 0; i < 3; ++i) {
        if (overlaps(outs[i], olen[i], x, nx) || overlaps(outs[i], olen[i], w, nw)) return ATTN_ERR_ALIAS;
        for (int j = i + 1; j < 3; ++j)
            if (overlaps(outs[i], olen[i], outs[j], olen[j])) return ATTN_ERR_ALIAS;
    }
    attn::QkvArgs a{};
    a.x = x;
    a.w = w;
    a.q = q;
    a.k = k;
    a.v = v;
    a.M = (int)M;
    a.N = (int)N;
    a.d_model = d_model;
    a.T = T;
    a.H_q = H_q;
    a.H_kv = H_kv;
    a.D = D;
    return hip_status(attn::launch_qkv_bf16(a, static_cast<hipStream_t>(stream)));
}

const char* attn_status_string(int status) {
    switch (status) {
        case ATTN_OK: return "ok";
        case ATTN_ERR_NULL_PTR: return "null pointer";
        case ATTN_ERR_INVALID_SHAPE: return "invalid shape";
        case ATTN_ERR_UNSUPPORTED: return "unsupported configuration";
        case ATTN_ERR_INVALID_SCALE: return "scale is not finite";
        case ATTN_ERR_ALIGNMENT: return "pointer not 16-byte aligned";
        case ATTN_ERR_ALIAS: return "output overlaps an input or the workspace";
        case ATTN_ERR_WORKSPACE: return "decode workspace missing or too small";
        case ATTN_ERR_HIP: return "HIP launch failed";
        case ATTN_ERR_SCRATCH: return "decode needs more scratch than the no-allocation entry point holds";
        default: return "unknown status";
    }
}

int attn_abi_version(void) { return ATTN_ABI_VERSION; }

int attn_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
