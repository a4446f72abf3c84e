// C ABI of libattn.so: argument validation and dispatch to the HIP launchers.
// Every check runs before the first HIP call, so a rejected request enqueues
// nothing and writes nothing.
#include <math.h>
#include <stdint.h>

#include <atomic>

#include "../../include/attn.h"
#include "attn_launch.h"

// Device scratch of attn_bwd_noalloc: the backward's one workspace buffer (the fp32 D
// rows, B*H*N floats) as a static array, so that entry point never allocates.  Each GPU
// holds its own copy until the process ends; host code reaches it only through the
// address hipGetSymbolAddress returns for the current device (the array's name is a
// host-side stand-in, not a device address).
static constexpr size_t kNoAllocRows = (size_t)ATTN_NOALLOC_MAX_ROWS;
static __device__ __align__(256) float scratch[kNoAllocRows];

namespace {

thread_local int g_last_hip_error = 0;

// Per-device address of `scratch`, looked up once per device with that device current.
constexpr int kMaxDevices = 64;
std::atomic<float*> g_scratch_ptr[kMaxDevices];

hipError_t scratch_for_current_device(float** out)
{
    int dev = 0;
    if (hipError_t e = hipGetDevice(&dev); e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    float* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        void* ptr = nullptr;
        if (hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)); e != hipSuccess) return e;
        if (ptr == nullptr) return hipErrorInvalidSymbol;
        p = static_cast<float*>(ptr);
        g_scratch_ptr[dev].store(p, std::memory_order_release);   // same value whichever thread wins
    }
    *out = p;
    return hipSuccess;
}

bool aligned16(const void* p) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

attn_status check_shape(int B, int H, int N, int d)
{
    if (B < 1 || H < 1 || N < 1 || d < 1) return ATTN_EINVAL;
    // one head's fp32 rows must stay below 2 GiB: the kernels address inside a head
    // with 32-bit byte offsets (heads themselves with 64-bit ones) and use 2^31 as
    // their out-of-range offset
    if ((long long)N * d * 4 >= (1LL << 31)) return ATTN_EINVAL;
    // the largest grid (one 512-thread workgroup per 128 rows of every head) must
    // stay below 2^32 work-items, the dispatch packet's limit
    if ((long long)B * H * ((N + 127) / 128) >= (1LL << 23)) return ATTN_EINVAL;
    if (d != 64 && d != 80 && d != 128) return ATTN_EUNSUPPORTED;
    return ATTN_OK;
}

bool dtype_ok(attn_dtype dt) { return dt == ATTN_F32 || dt == ATTN_BF16; }

attn_status from_hip(hipError_t e)
{
    if (e == hipSuccess) return ATTN_OK;
    g_last_hip_error = (int)e;
    return ATTN_EHIP;
}

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

extern "C" {

const char* attn_status_str(attn_status s)
{
    switch (s) {
        case ATTN_OK: return "ok";
        case ATTN_EINVAL: return "invalid argument";
        case ATTN_EUNSUPPORTED: return "unsupported configuration";
        case ATTN_EHIP: return "HIP runtime error";
        case ATTN_ENOSPACE: return "request exceeds the static scratch of the allocation-free entry point";
    }
    return "unknown status";
}

int attn_last_hip_error(void) { return g_last_hip_error; }

attn_status attn_fwd(const void* Q, const void* K, const void* V, attn_dtype dt, int B, int H, int N, int d,
                     float scale, int causal, void* O, float* LSE, void* stream)
{
    attn_status s = check_shape(B, H, N, d);
    if (s != ATTN_OK) return s;
    if (!dtype_ok(dt) || !isfinite(scale) || (causal != 0 && causal != 1)) return ATTN_EINVAL;
    if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(LSE)) return ATTN_EINVAL;
    return from_hip(attn::launch_fwd(Q, K, V, O, LSE, dt == ATTN_BF16, B * H, N, d, scale, causal, nullptr, 0,
                                     (hipStream_t)stream));
}

attn_status attn_bwd_preprocess(const void* O, const void* dO, attn_dtype dt, int B, int H, int N, int d,
                                float* D, void* stream)
{
    attn_status s = check_shape(B, H, N, d);
    if (s != ATTN_OK) return s;
    if (!dtype_ok(dt)) return ATTN_EINVAL;
    if (!aligned16(O) || !aligned16(dO) || !aligned16(D)) return ATTN_EINVAL;
    return from_hip(attn::launch_bwd_pre(O, dO, dt == ATTN_BF16, B * H, N, d, D, (hipStream_t)stream));
}

static attn_status check_bwd_args(const void* Q, const void* K, const void* V, const void* dO, const float* LSE,
                                  const float* D, attn_dtype dt, int B, int H, int N, int d, float scale, int causal)
{
    attn_status s = check_shape(B, H, N, d);
    if (s != ATTN_OK) return s;
    if (!dtype_ok(dt) || !isfinite(scale) || (causal != 0 && causal != 1)) return ATTN_EINVAL;
    if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(dO) || !aligned16(LSE) || !aligned16(D))
        return ATTN_EINVAL;
    return ATTN_OK;
}

attn_status attn_bwd_dkdv(const void* Q, const void* K, const void* V, const void* dO, const float* LSE,
                          const float* D, attn_dtype dt, int B, int H, int N, int d, float scale, int causal,
                          float* dK, float* dV, void* stream)
{
    attn_status s = check_bwd_args(Q, K, V, dO, LSE, D, dt, B, H, N, d, scale, causal);
    if (s != ATTN_OK) return s;
    if (!aligned16(dK) || !aligned16(dV)) return ATTN_EINVAL;
    if (dt != ATTN_BF16) return ATTN_EUNSUPPORTED;
    return from_hip(attn::launch_bwd_dkdv(Q, K, V, dO, LSE, D, B * H, N, d, scale, causal, dK, dV, false, nullptr,
                                          0, (hipStream_t)stream));
}

attn_status attn_bwd_dq(const void* Q, const void* K, const void* V, const void* dO, const float* LSE,
                        const float* D, attn_dtype dt, int B, int H, int N, int d, float scale, int causal,
                        float* dQ, void* stream)
{
    attn_status s = check_bwd_args(Q, K, V, dO, LSE, D, dt, B, H, N, d, scale, causal);
    if (s != ATTN_OK) return s;
    if (!aligned16(dQ)) return ATTN_EINVAL;
    if (dt != ATTN_BF16) return ATTN_EUNSUPPORTED;
    return from_hip(attn::launch_bwd_dq(Q, K, V, dO, LSE, const_cast<float*>(D), nullptr, B * H, N, d, scale,
                                        causal, dQ, false, nullptr, 0, (hipStream_t)stream));
}

attn_status attn_bwd_dq_d(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                          const float* LSE, attn_dtype dt, int B, int H, int N, int d, float scale, int causal,
                          float* D, float* dQ, void* stream)
{
    attn_status s = check_bwd_args(Q, K, V, dO, LSE, D, dt, B, H, N, d, scale, causal);
    if (s != ATTN_OK) return s;
    if (!aligned16(O) || !aligned16(dQ)) return ATTN_EINVAL;
    if (dt != ATTN_BF16) return ATTN_EUNSUPPORTED;
    return from_hip(attn::launch_bwd_dq(Q, K, V, dO, LSE, D, O, B * H, N, d, scale, causal, dQ, false, nullptr, 0,
                                        (hipStream_t)stream));
}

attn_status attn_bwd_main(const void* Q, const void* K, const void* V, const void* dO, const float* LSE,
                          const float* D, attn_dtype dt, int B, int H, int N, int d, float scale, int causal,
                          float* dQ, float* dK, float* dV, void* stream)
{
    attn_status s = check_bwd_args(Q, K, V, dO, LSE, D, dt, B, H, N, d, scale, causal);
    if (s != ATTN_OK) return s;
    if (!aligned16(dQ) || !aligned16(dK) || !aligned16(dV)) return ATTN_EINVAL;
    hipStream_t st = (hipStream_t)stream;
    if (dt == ATTN_F32)
        return from_hip(attn::launch_bwd_f32(Q, K, V, dO, LSE, D, B * H, N, d, scale, causal, dQ, dK, dV, nullptr, 0,
                                             st));
    attn_status r = from_hip(attn::launch_bwd_dkdv(Q, K, V, dO, LSE, D, B * H, N, d, scale, causal, dK, dV, false,
                                                   nullptr, 0, st));
    if (r != ATTN_OK) return r;
    return from_hip(attn::launch_bwd_dq(Q, K, V, dO, LSE, const_cast<float*>(D), nullptr, B * H, N, d, scale, causal,
                                        dQ, false, nullptr, 0, st));
}

size_t attn_bwd_workspace_bytes(int B, int H, int N, int d, attn_dtype grad_dt)
{
    if (check_shape(B, H, N, d) == ATTN_EINVAL || !dtype_ok(grad_dt)) return 0;
    // D only: every gradient is written once in its own dtype (dQ by the query-side
    // kernel, or for fp32 inputs accumulated in place in the fp32 dQ), so no fp32
    // staging of bf16 gradients is needed
    return round256((size_t)B * H * N * sizeof(float));
}

static attn_status bwd_all(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                           const float* LSE, attn_dtype dt, int B, int H, int N, int d, float scale, int causal,
                           const unsigned char* bmask, long mhead, void* dQ, void* dK, void* dV,
                           attn_dtype grad_dt, void* workspace, size_t workspace_bytes, void* stream)
{
    attn_status s = check_bwd_args(Q, K, V, dO, LSE, (const float*)workspace, dt, B, H, N, d, scale, causal);
    if (s != ATTN_OK) return s;
    if (!dtype_ok(grad_dt)) return ATTN_EINVAL;
    if (!aligned16(O) || !aligned16(dQ) || !aligned16(dK) || !aligned16(dV)) return ATTN_EINVAL;
    if (workspace_bytes < attn_bwd_workspace_bytes(B, H, N, d, grad_dt)) return ATTN_EINVAL;
    if (dt == ATTN_F32 && grad_dt == ATTN_BF16) return ATTN_EUNSUPPORTED;

    hipStream_t st = (hipStream_t)stream;
    const bool bf_in = dt == ATTN_BF16, bf_grad = grad_dt == ATTN_BF16;
    const int BH = B * H;
    float* Dd = static_cast<float*>(workspace);
    if (!bf_in) {
        attn_status r = from_hip(attn::launch_bwd_pre(O, dO, bf_in, BH, N, d, Dd, st));
        if (r != ATTN_OK) return r;
        return from_hip(attn::launch_bwd_f32(Q, K, V, dO, LSE, Dd, BH, N, d, scale, causal, (float*)dQ, (float*)dK,
                                             (float*)dV, bmask, mhead, st));
    }
    // bf16: the dQ kernel also computes D (the preprocess) for its rows; the key side reads it
    attn_status r = from_hip(attn::launch_bwd_dq(Q, K, V, dO, LSE, Dd, O, BH, N, d, scale, causal, dQ, bf_grad, bmask,
                                                 mhead, st));
    if (r != ATTN_OK) return r;
    return from_hip(attn::launch_bwd_dkdv(Q, K, V, dO, LSE, Dd, BH, N, d, scale, causal, dK, dV, bf_grad, bmask,
                                          mhead, st));
}

attn_status attn_bwd(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                     const float* LSE, attn_dtype dt, int B, int H, int N, int d, float scale, int causal,
                     void* dQ, void* dK, void* dV, attn_dtype grad_dt, void* workspace,
                     size_t workspace_bytes, void* stream)
{
    return bwd_all(Q, K, V, O, dO, LSE, dt, B, H, N, d, scale, causal, nullptr, 0, dQ, dK, dV, grad_dt, workspace,
                   workspace_bytes, stream);
}

attn_status attn_bwd_noalloc(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                             const float* LSE, attn_dtype dt, int B, int H, int N, int d, float scale, int causal,
                             void* dQ, void* dK, void* dV, attn_dtype grad_dt, void* stream)
{
    attn_status s = check_shape(B, H, N, d);
    if (s != ATTN_OK) return s;
    if ((size_t)B * (size_t)H * (size_t)N > kNoAllocRows) return ATTN_ENOSPACE;
    float* ws = nullptr;
    if (attn_status r = from_hip(scratch_for_current_device(&ws)); r != ATTN_OK) return r;
    return bwd_all(Q, K, V, O, dO, LSE, dt, B, H, N, d, scale, causal, nullptr, 0, dQ, dK, dV, grad_dt, ws,
                   kNoAllocRows * sizeof(float), stream);
}

attn_status attn_fwd_fp8(const void* Q, const void* K, const void* V, float q_descale, float k_descale,
                         float v_descale, int B, int H, int N, int d, float scale, int causal, void* O, float* LSE,
                         void* stream)
{
    attn_status s = check_shape(B, H, N, d);
    if (s != ATTN_OK) return s;
    if (d == 80) return ATTN_EUNSUPPORTED;
    if (!isfinite(scale) || !isfinite(q_descale) || !isfinite(k_descale) || !isfinite(v_descale) ||
        (causal != 0 && causal != 1))
        return ATTN_EINVAL;
    if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(LSE)) return ATTN_EINVAL;
    return from_hip(attn::launch_fwd_fp8(Q, K, V, q_descale, k_descale, v_descale, O, LSE, B * H, N, d, scale, causal,
                                         (hipStream_t)stream));
}

// bytes between the masks of consecutive heads, or -1 for a bad mask argument
static long mask_head_stride(const unsigned char* block_mask, int mask_heads, int B, int H, int N)
{
    if (block_mask == nullptr) return -1;
    if (mask_heads != 1 && (long long)mask_heads != (long long)B * H) return -1;
    const long T = (N + ATTN_MASK_BLOCK - 1) / ATTN_MASK_BLOCK;
    return mask_heads == 1 ? 0 : T * T;
}

attn_status attn_fwd_blocksparse(const void* Q, const void* K, const void* V, attn_dtype dt, int B, int H, int N,
                                 int d, float scale, int causal, const unsigned char* block_mask, int mask_heads,
                                 void* O, float* LSE, void* stream)
{
    attn_status s = check_shape(B, H, N, d);
    if (s != ATTN_OK) return s;
    if (!dtype_ok(dt) || !isfinite(scale) || (causal != 0 && causal != 1)) return ATTN_EINVAL;
    if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(LSE)) return ATTN_EINVAL;
    const long mhead = mask_head_stride(block_mask, mask_heads, B, H, N);
    if (mhead < 0) return ATTN_EINVAL;
    return from_hip(attn::launch_fwd(Q, K, V, O, LSE, dt == ATTN_BF16, B * H, N, d, scale, causal, block_mask,
                                     mhead, (hipStream_t)stream));
}

attn_status attn_bwd_blocksparse(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                                 const float* LSE, attn_dtype dt, int B, int H, int N, int d, float scale,
                                 int causal, const unsigned char* block_mask, int mask_heads, void* dQ, void* dK,
                                 void* dV, attn_dtype grad_dt, void* workspace, size_t workspace_bytes,
                                 void* stream)
{
    const long mhead = mask_head_stride(block_mask, mask_heads, B, H, N);
    if (mhead < 0) return ATTN_EINVAL;
    return bwd_all(Q, K, V, O, dO, LSE, dt, B, H, N, d, scale, causal, block_mask, mhead, dQ, dK, dV, grad_dt,
                   workspace, workspace_bytes, stream);
}

}  // extern "C"
