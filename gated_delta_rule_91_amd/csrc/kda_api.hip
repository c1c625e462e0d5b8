// kda_api.hip -- the C ABI of libkda.so (declared in include/kda.h).
//
// Every entry point validates its arguments synchronously, before any
// launch, maps them to the kernel argument blocks and launches on the
// caller's stream.  Nothing here allocates.  The only state is the fixed
// scratch area of kda_prefill_noalloc (below) and its per-device address.
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "kda.h"
#include "kda_internal.hpp"

using namespace kda;

// Update cards of kda_prefill_noalloc.  Each GPU the library runs on holds
// its own copy until the process ends.  Host code never uses this name as a
// device address (on the host it is only a stand-in for the symbol): the
// address of the current device's copy comes from hipGetSymbolAddress, once
// per device, and only that address reaches kernels.
static __device__ __align__(256) unsigned char scratch[KDA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices] = {};

// Device address of the current device's scratch array, looked up on the
// first call on that device (with that device current) and kept.
kda_status scratch_address(void** addr) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return KDA_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return KDA_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_addr[dev]) {
        void* a = nullptr;
        if (hipGetSymbolAddress(&a, HIP_SYMBOL(scratch)) != hipSuccess || a == nullptr) return KDA_ERR_HIP;
        g_scratch_addr[dev] = a;
    }
    *addr = g_scratch_addr[dev];
    return KDA_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// ptr must be non-null and 16-byte aligned when the array is non-empty
bool ok_ptr(const void* p, bool nonempty) { return !nonempty || (p != nullptr && aligned16(p)); }
// beta is only read one fp32 at a time: natural alignment suffices
bool ok_beta(const void* p, bool nonempty) { return !nonempty || (p != nullptr && ((uintptr_t)p & 3u) == 0); }
bool ok_opt_ptr(const void* p) { return p == nullptr || aligned16(p); }

kda_status check_floor(float f, int chunk) {
    // the floor keeps exp(chunk * |floor|) -- the largest decay factor folded
    // into one chunk's operands -- below e^80, inside fp32/bf16 range
    if (!(f < 0.0f) || !(f >= -80.0f / (float)chunk)) return KDA_ERR_INVALID_ARGUMENT;
    return KDA_OK;
}

kda_status check_problem(const kda_problem* p) {
    if (!p) return KDA_ERR_INVALID_ARGUMENT;
    if (p->batch < 0 || p->seqlen < 0 || p->heads <= 0 || p->dk <= 0 || p->dv <= 0 || p->chunk <= 0)
        return KDA_ERR_INVALID_ARGUMENT;
    if (p->io_dtype != KDA_F32 && p->io_dtype != KDA_BF16) return KDA_ERR_INVALID_ARGUMENT;
    if (p->chunk != 64) return KDA_ERR_UNSUPPORTED;
    if (p->dk != p->dv || (p->dk != 64 && p->dk != 128)) return KDA_ERR_UNSUPPORTED;
    const kda_status f = check_floor(p->log_alpha_min, p->chunk);
    if (f != KDA_OK) return f;
    const int64_t nc = (p->seqlen + p->chunk - 1) / p->chunk;
    // grid sizes and offsets must fit the kernels' index arithmetic
    if (p->batch * (int64_t)p->heads * (nc > 0 ? nc : 1) > (int64_t)INT32_MAX) return KDA_ERR_UNSUPPORTED;
    if (nc > (int64_t)INT32_MAX) return KDA_ERR_UNSUPPORTED;
    return KDA_OK;
}

int64_t n_chunks(const kda_problem* p) { return (p->seqlen + p->chunk - 1) / p->chunk; }

kda_status device_ready() {
    int dev = 0;
    return hipGetDevice(&dev) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status hip_status(hipError_t e) { return e == hipSuccess ? KDA_OK : KDA_ERR_HIP; }

// Packed variable-length batches: chunk offsets first, then each chunk's
// sequence index, then the cards.
size_t varlen_offsets_bytes(int64_t n_seq) { return ((size_t)(n_seq + 1) * 8 + 255) / 256 * 256; }
int64_t varlen_max_chunks(const kda_problem* p, int64_t n_seq) { return n_chunks(p) + n_seq; }
size_t varlen_seqmap_bytes(const kda_problem* p, int64_t n_seq) {
    return ((size_t)varlen_max_chunks(p, n_seq) * 4 + 255) / 256 * 256;
}
size_t varlen_cards_offset(const kda_problem* p, int64_t n_seq) {
    return varlen_offsets_bytes(n_seq) + varlen_seqmap_bytes(p, n_seq);
}

kda_status check_varlen(const kda_problem* p, int64_t n_seq) {
    kda_status st = check_problem(p);
    if (st != KDA_OK) return st;
    if (p->batch != 1 || n_seq < 0) return KDA_ERR_INVALID_ARGUMENT;
    if ((varlen_max_chunks(p, n_seq) + 1) * (int64_t)p->heads > (int64_t)INT32_MAX) return KDA_ERR_UNSUPPORTED;
    if (n_seq * (int64_t)p->heads * (p->dv / 16) > (int64_t)INT32_MAX) return KDA_ERR_UNSUPPORTED;
    return KDA_OK;
}

// Launch arguments for chunks [c0, c1) of every (row, head) of a uniform
// batch: the range's first token rows inside the whole [B, T, H, d] arrays
// (rows stay T tokens apart), its cards at `cards`.  The caller sets the
// scan's state_in and state_out.
struct RangeLaunch {
    PrepareArgs pa;
    ScanArgs sa;
};
RangeLaunch range_launch(const kda_problem* p, const void* q, const void* k, const void* v, const float* log_alpha,
                         const float* beta, const void* g, void* out, char* cards, int64_t c0, int64_t c1) {
    const size_t esz = p->io_dtype == KDA_BF16 ? 2 : 4;
    const int64_t T = p->seqlen;
    const int64_t t0 = c0 * p->chunk, t1 = c1 * p->chunk < T ? c1 * p->chunk : T;
    const size_t tok = (size_t)t0 * (size_t)p->heads;   // row-0 offset of the range, in token-heads
    RangeLaunch r = {};
    r.pa.q = static_cast<const char*>(q) + tok * p->dk * esz;
    r.pa.k = static_cast<const char*>(k) + tok * p->dk * esz;
    r.pa.v = static_cast<const char*>(v) + tok * p->dv * esz;
    r.pa.log_alpha = log_alpha + tok * p->dk;
    r.pa.beta = beta + tok;
    r.pa.ws = cards;
    r.pa.B = p->batch; r.pa.T = t1 - t0; r.pa.row_stride = T; r.pa.H = p->heads; r.pa.NC = (int)(c1 - c0);
    r.pa.floor_ = p->log_alpha_min;
    r.sa.ws = cards;
    r.sa.g = static_cast<const char*>(g) + tok * p->dv * esz;
    r.sa.out = static_cast<char*>(out) + tok * p->dv * esz;
    r.sa.B = p->batch; r.sa.T = t1 - t0; r.sa.row_stride = T; r.sa.H = p->heads; r.sa.NC = (int)(c1 - c0);
    return r;
}

// No tokens: state_out = state_in (or zero), through the scan kernel.
kda_status copy_state(const kda_problem* p, const float* state_in, float* state_out, hipStream_t s) {
    ScanArgs a = {};
    a.state_in = state_in; a.state_out = state_out;
    a.B = p->batch; a.T = 0; a.H = p->heads; a.NC = 0;
    return hip_status(launch_scan(p->io_dtype == KDA_BF16, p->dk, false, a, s));
}

// The pipelined prefill's workspace: the carried state, then one or two
// ranges' cards.
size_t state_bytes_of(const kda_problem* p) {
    return ((size_t)p->batch * (size_t)p->heads * (size_t)p->dk * (size_t)p->dv * 4 + 255) / 256 * 256;
}
int64_t range_of(const kda_problem* p, int32_t range_chunks) {
    const int64_t nc = n_chunks(p);
    return range_chunks < nc ? range_chunks : nc;
}
size_t range_card_bytes(const kda_problem* p, int64_t rc) {
    return ((size_t)rc * (size_t)p->batch * (size_t)p->heads * card_bytes(p->io_dtype == KDA_BF16, p->dk) + 255) /
           256 * 256;
}

}  // namespace

extern "C" {

const char* kda_status_string(kda_status s) {
    switch (s) {
        case KDA_OK: return "ok";
        case KDA_ERR_INVALID_ARGUMENT: return "invalid argument";
        case KDA_ERR_UNSUPPORTED: return "unsupported shape or dtype";
        case KDA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
        case KDA_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

size_t kda_workspace_size(const kda_problem* p) {
    if (check_problem(p) != KDA_OK) return 0;
    return (size_t)p->batch * (size_t)p->heads * (size_t)n_chunks(p) * card_bytes(p->io_dtype == KDA_BF16, p->dk);
}

kda_status kda_chunk_prepare(const kda_problem* p, const void* q, const void* k, const void* v,
                             const float* log_alpha, const float* beta, void* workspace, size_t workspace_bytes,
                             void* stream) {
    kda_status st = check_problem(p);
    if (st != KDA_OK) return st;
    const bool nonempty = p->batch > 0 && p->seqlen > 0;
    if (!ok_ptr(q, nonempty) || !ok_ptr(k, nonempty) || !ok_ptr(v, nonempty) || !ok_ptr(log_alpha, nonempty) ||
        !ok_beta(beta, nonempty) || !ok_ptr(workspace, nonempty))
        return KDA_ERR_INVALID_ARGUMENT;
    if (workspace_bytes < kda_workspace_size(p)) return KDA_ERR_WORKSPACE_TOO_SMALL;
    if (!nonempty) return KDA_OK;
    if ((st = device_ready()) != KDA_OK) return st;
    PrepareArgs a = {};
    a.q = q; a.k = k; a.v = v; a.log_alpha = log_alpha; a.beta = beta;
    a.ws = static_cast<char*>(workspace);
    a.B = p->batch; a.T = p->seqlen; a.H = p->heads; a.NC = (int)n_chunks(p);
    a.floor_ = p->log_alpha_min;
    return hip_status(launch_prepare(p->io_dtype == KDA_BF16, p->dk, a, (hipStream_t)stream));
}

kda_status kda_chunk_scan(const kda_problem* p, const void* workspace, size_t workspace_bytes, const void* g,
                          const float* state_in, void* out, float* state_out, void* stream) {
    kda_status st = check_problem(p);
    if (st != KDA_OK) return st;
    const bool tokens = p->batch > 0 && p->seqlen > 0;
    if (!ok_ptr(workspace, tokens) || !ok_ptr(g, tokens) || !ok_ptr(out, tokens) || !ok_opt_ptr(state_in) ||
        !ok_opt_ptr(state_out))
        return KDA_ERR_INVALID_ARGUMENT;
    if (workspace_bytes < kda_workspace_size(p)) return KDA_ERR_WORKSPACE_TOO_SMALL;
    if (p->batch == 0 || (!tokens && !state_out)) return KDA_OK;
    if ((st = device_ready()) != KDA_OK) return st;
    ScanArgs a = {};
    a.ws = static_cast<const char*>(workspace);
    a.g = g; a.state_in = state_in; a.out = out; a.state_out = state_out;
    a.B = p->batch; a.T = p->seqlen; a.H = p->heads; a.NC = (int)n_chunks(p);
    return hip_status(launch_scan(p->io_dtype == KDA_BF16, p->dk, false, a, (hipStream_t)stream));
}

kda_status kda_chunk_scan_checkpoints(const kda_problem* p, const void* workspace, size_t workspace_bytes,
                                      const void* g, const float* state_in, void* out, float* state_out,
                                      int32_t every, float* checkpoints, void* stream) {
    kda_status st = check_problem(p);
    if (st != KDA_OK) return st;
    if (every < 1) return KDA_ERR_INVALID_ARGUMENT;
    const bool tokens = p->batch > 0 && p->seqlen > 0;
    if (!ok_ptr(workspace, tokens) || !ok_ptr(g, tokens) || !ok_ptr(out, tokens) || !ok_opt_ptr(state_in) ||
        !ok_opt_ptr(state_out) || !ok_ptr(checkpoints, p->batch > 0))
        return KDA_ERR_INVALID_ARGUMENT;
    if (workspace_bytes < kda_workspace_size(p)) return KDA_ERR_WORKSPACE_TOO_SMALL;
    if (p->batch == 0) return KDA_OK;
    if ((st = device_ready()) != KDA_OK) return st;
    // every >= NC gives the same slots as every == NC (entry 0 and the final
    // state), so clamping keeps the kernel's slot arithmetic small
    const int64_t nc = n_chunks(p);
    if ((int64_t)every > nc) every = (int32_t)(nc > 1 ? nc : 1);
    ScanArgs a = {};
    a.ws = static_cast<const char*>(workspace);
    a.g = g; a.state_in = state_in; a.out = out; a.state_out = state_out;
    a.states = checkpoints; a.ckpt_every = every;
    a.B = p->batch; a.T = p->seqlen; a.H = p->heads; a.NC = (int)n_chunks(p);
    return hip_status(launch_scan(p->io_dtype == KDA_BF16, p->dk, false, a, (hipStream_t)stream));
}

kda_status kda_segment_summarize(const kda_problem* p, const void* workspace, size_t workspace_bytes,
                                 float* transition, float* zero_state, void* stream) {
    kda_status st = check_problem(p);
    if (st != KDA_OK) return st;
    const bool rows = p->batch > 0;
    if (!ok_ptr(workspace, rows && p->seqlen > 0) || !ok_ptr(transition, rows) || !ok_ptr(zero_state, rows))
        return KDA_ERR_INVALID_ARGUMENT;
    if (workspace_bytes < kda_workspace_size(p)) return KDA_ERR_WORKSPACE_TOO_SMALL;
    if (!rows) return KDA_OK;
    if ((st = device_ready()) != KDA_OK) return st;
    ScanArgs a = {};
    a.ws = static_cast<const char*>(workspace);
    a.transition = transition; a.zero_state = zero_state;
    a.B = p->batch; a.T = p->seqlen; a.H = p->heads; a.NC = (int)n_chunks(p);
    return hip_status(launch_scan(p->io_dtype == KDA_BF16, p->dk, true, a, (hipStream_t)stream));
}

kda_status kda_segment_combine(int64_t B, int32_t n_seg, int32_t H, int32_t dk, int32_t dv, const float* transition,
                               const float* zero_state, const float* state_init, float* seg_state_in,
                               float* state_final, void* stream) {
    if (B < 0 || n_seg < 0 || H <= 0 || dk <= 0 || dv <= 0) return KDA_ERR_INVALID_ARGUMENT;
    if (dk != dv || (dk != 64 && dk != 128)) return KDA_ERR_UNSUPPORTED;
    if (B * (int64_t)H * (dv / 16) > (int64_t)INT32_MAX) return KDA_ERR_UNSUPPORTED;
    const bool segs = B > 0 && n_seg > 0;
    if (!ok_ptr(transition, segs) || !ok_ptr(zero_state, segs) || !ok_ptr(seg_state_in, segs) ||
        !ok_opt_ptr(state_init) || !ok_opt_ptr(state_final))
        return KDA_ERR_INVALID_ARGUMENT;
    if (B == 0 || (n_seg == 0 && !state_final)) return KDA_OK;
    kda_status st = device_ready();
    if (st != KDA_OK) return st;
    CombineArgs a;
    a.A = transition; a.Bz = zero_state; a.s0 = state_init; a.seg_in = seg_state_in; a.fin = state_final;
    a.B = B; a.n_seg = n_seg; a.H = H; a.dk = dk; a.dv = dv;
    return hip_status(launch_combine(a, (hipStream_t)stream));
}

kda_status kda_decode_step(int64_t N, int32_t H, int32_t dk, int32_t dv, kda_dtype io_dtype, float log_alpha_min,
                           const void* q, const void* k, const void* v, const float* log_alpha, const float* beta,
                           const void* g, float* state, void* out, void* stream) {
    if (N < 0 || H <= 0 || dk <= 0 || dv <= 0) return KDA_ERR_INVALID_ARGUMENT;
    if (io_dtype != KDA_F32 && io_dtype != KDA_BF16) return KDA_ERR_INVALID_ARGUMENT;
    if (dk != dv || (dk != 64 && dk != 128)) return KDA_ERR_UNSUPPORTED;
    if (N * (int64_t)H > (int64_t)INT32_MAX) return KDA_ERR_UNSUPPORTED;
    kda_status st = check_floor(log_alpha_min, 64);
    if (st != KDA_OK) return st;
    const bool any = N > 0;
    if (!ok_ptr(q, any) || !ok_ptr(k, any) || !ok_ptr(v, any) || !ok_ptr(log_alpha, any) || !ok_beta(beta, any) ||
        !ok_ptr(g, any) || !ok_ptr(state, any) || !ok_ptr(out, any))
        return KDA_ERR_INVALID_ARGUMENT;
    if (!any) return KDA_OK;
    if ((st = device_ready()) != KDA_OK) return st;
    DecodeArgs a;
    a.q = q; a.k = k; a.v = v; a.log_alpha = log_alpha; a.beta = beta; a.g = g; a.state = state; a.out = out;
    a.N = N; a.H = H; a.floor_ = log_alpha_min;
    return hip_status(launch_decode(io_dtype == KDA_BF16, dk, a, (hipStream_t)stream));
}

size_t kda_varlen_workspace_size(const kda_problem* p, int64_t n_seq) {
    if (check_varlen(p, n_seq) != KDA_OK || n_seq == 0) return 0;
    return varlen_cards_offset(p, n_seq) +
           (size_t)varlen_max_chunks(p, n_seq) * (size_t)p->heads * card_bytes(p->io_dtype == KDA_BF16, p->dk);
}

kda_status kda_varlen_prepare(const kda_problem* p, int64_t n_seq, const int32_t* cu_seqlens, const void* q,
                              const void* k, const void* v, const float* log_alpha, const float* beta,
                              void* workspace, size_t workspace_bytes, void* stream) {
    kda_status st = check_varlen(p, n_seq);
    if (st != KDA_OK) return st;
    const bool tokens = p->seqlen > 0;
    if (!ok_beta(cu_seqlens, n_seq > 0) || !ok_ptr(q, tokens) || !ok_ptr(k, tokens) || !ok_ptr(v, tokens) ||
        !ok_ptr(log_alpha, tokens) || !ok_beta(beta, tokens) || !ok_ptr(workspace, n_seq > 0))
        return KDA_ERR_INVALID_ARGUMENT;
    if (workspace_bytes < kda_varlen_workspace_size(p, n_seq)) return KDA_ERR_WORKSPACE_TOO_SMALL;
    if (n_seq == 0) return KDA_OK;
    if ((st = device_ready()) != KDA_OK) return st;
    PrepareArgs a = {};
    a.q = q; a.k = k; a.v = v; a.log_alpha = log_alpha; a.beta = beta;
    a.chunk_off = static_cast<int64_t*>(workspace);
    a.chunk_seq = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + varlen_offsets_bytes(n_seq));
    a.ws = static_cast<char*>(workspace) + varlen_cards_offset(p, n_seq);
    a.cu_seqlens = cu_seqlens;
    a.B = n_seq; a.T = p->seqlen; a.H = p->heads; a.NC = 0;
    a.floor_ = p->log_alpha_min;
    return hip_status(launch_prepare(p->io_dtype == KDA_BF16, p->dk, a, (hipStream_t)stream));
}

kda_status kda_varlen_scan(const kda_problem* p, int64_t n_seq, const int32_t* cu_seqlens, const void* workspace,
                           size_t workspace_bytes, const void* g, const float* state_in, void* out, float* state_out,
                           void* stream) {
    kda_status st = check_varlen(p, n_seq);
    if (st != KDA_OK) return st;
    const bool tokens = p->seqlen > 0;
    if (!ok_beta(cu_seqlens, n_seq > 0) || !ok_ptr(workspace, n_seq > 0) || !ok_ptr(g, tokens) ||
        !ok_ptr(out, tokens) || !ok_opt_ptr(state_in) || !ok_opt_ptr(state_out))
        return KDA_ERR_INVALID_ARGUMENT;
    if (workspace_bytes < kda_varlen_workspace_size(p, n_seq)) return KDA_ERR_WORKSPACE_TOO_SMALL;
    if (n_seq == 0 || (!tokens && !state_out)) return KDA_OK;
    if ((st = device_ready()) != KDA_OK) return st;
    ScanArgs a = {};
    a.chunk_off = static_cast<const int64_t*>(workspace);
    a.ws = static_cast<const char*>(workspace) + varlen_cards_offset(p, n_seq);
    a.cu_seqlens = cu_seqlens;
    a.g = g; a.state_in = state_in; a.out = out; a.state_out = state_out;
    a.B = n_seq; a.T = p->seqlen; a.H = p->heads; a.NC = 0;
    return hip_status(launch_scan(p->io_dtype == KDA_BF16, p->dk, false, a, (hipStream_t)stream));
}

size_t kda_backward_workspace_size(const kda_problem* p) {
    if (check_problem(p) != KDA_OK || p->seqlen == 0) return 0;
    return backward_workspace_bytes(p->io_dtype == KDA_BF16, p->batch, p->seqlen, p->heads, p->dk);
}

// Argument checks and the launch arguments shared by kda_backward and
// kda_backward_after_prefill.
static kda_status backward_args(const kda_problem* p, const void* q, const void* k, const void* v,
                                const float* log_alpha, const float* beta, const void* g, const float* state_in,
                                const void* out, bool need_out, const void* d_out, const float* d_state, void* dq,
                                void* dk, void* dv, float* dlog_alpha, float* dbeta, void* dg, float* d_state_in,
                                void* workspace, size_t workspace_bytes, BackwardArgs* a, bool* work) {
    kda_status st = check_problem(p);
    if (st != KDA_OK) return st;
    const bool tokens = p->batch > 0 && p->seqlen > 0;
    if (!ok_ptr(q, tokens) || !ok_ptr(k, tokens) || !ok_ptr(v, tokens) || !ok_ptr(log_alpha, tokens) ||
        !ok_beta(beta, tokens) || !ok_ptr(g, tokens) || !ok_ptr(dq, tokens) || !ok_ptr(dk, tokens) ||
        !ok_ptr(dv, tokens) || !ok_ptr(dlog_alpha, tokens) || !ok_beta(dbeta, tokens) || !ok_ptr(dg, tokens) ||
        !ok_ptr(workspace, tokens) || !ok_ptr(out, need_out && tokens) || !ok_opt_ptr(state_in) ||
        !ok_opt_ptr(d_out) || !ok_opt_ptr(d_state) || !ok_opt_ptr(d_state_in))
        return KDA_ERR_INVALID_ARGUMENT;
    if (workspace_bytes < kda_backward_workspace_size(p)) return KDA_ERR_WORKSPACE_TOO_SMALL;
    *work = !(p->batch == 0 || (!tokens && !d_state_in));
    if (!*work) return KDA_OK;
    if ((st = device_ready()) != KDA_OK) return st;
    a->q = q; a->k = k; a->v = v; a->log_alpha = log_alpha; a->beta = beta; a->g = g; a->state_in = state_in;
    a->d_out = d_out; a->d_state = d_state;
    a->dq = dq; a->dk = dk; a->dv = dv; a->dlog_alpha = dlog_alpha; a->dbeta = dbeta; a->dg = dg;
    a->d_state_in = d_state_in;
    a->out = out;
    a->ws = static_cast<char*>(workspace);
    a->B = p->batch; a->T = p->seqlen; a->H = p->heads; a->NC = (int)n_chunks(p); a->floor_ = p->log_alpha_min;
    return KDA_OK;
}

kda_status kda_backward(const kda_problem* p, const void* q, const void* k, const void* v, const float* log_alpha,
                        const float* beta, const void* g, const float* state_in, const void* d_out,
                        const float* d_state, void* dq, void* dk, void* dv, float* dlog_alpha, float* dbeta,
                        void* dg, float* d_state_in, void* workspace, size_t workspace_bytes, void* stream) {
    BackwardArgs a = {};
    bool work = false;
    const kda_status st = backward_args(p, q, k, v, log_alpha, beta, g, state_in, nullptr, false, d_out, d_state,
                                        dq, dk, dv, dlog_alpha, dbeta, dg, d_state_in, workspace, workspace_bytes,
                                        &a, &work);
    if (st != KDA_OK || !work) return st;
    return hip_status(launch_backward(p->io_dtype == KDA_BF16, p->dk, a, true, (hipStream_t)stream));
}

kda_status kda_prefill_for_backward(const kda_problem* p, const void* q, const void* k, const void* v,
                                    const float* log_alpha, const float* beta, const void* g,
                                    const float* state_in, void* out, float* state_out, void* workspace,
                                    size_t workspace_bytes, void* stream) {
    kda_status st = check_problem(p);
    if (st != KDA_OK) return st;
    const bool tokens = p->batch > 0 && p->seqlen > 0;
    if (!ok_ptr(q, tokens) || !ok_ptr(k, tokens) || !ok_ptr(v, tokens) || !ok_ptr(log_alpha, tokens) ||
        !ok_beta(beta, tokens) || !ok_ptr(g, tokens) || !ok_ptr(out, tokens) || !ok_ptr(workspace, tokens) ||
        !ok_opt_ptr(state_in) || !ok_opt_ptr(state_out))
        return KDA_ERR_INVALID_ARGUMENT;
    if (workspace_bytes < kda_backward_workspace_size(p)) return KDA_ERR_WORKSPACE_TOO_SMALL;
    if (p->batch == 0 || (!tokens && !state_out)) return KDA_OK;
    if ((st = device_ready()) != KDA_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    if (!tokens) return copy_state(p, state_in, state_out, s);
    BackwardArgs a = {};
    a.q = q; a.k = k; a.v = v; a.log_alpha = log_alpha; a.beta = beta; a.g = g; a.state_in = state_in;
    a.ws = static_cast<char*>(workspace);
    a.B = p->batch; a.T = p->seqlen; a.H = p->heads; a.NC = (int)n_chunks(p); a.floor_ = p->log_alpha_min;
    return hip_status(launch_backward_forward(p->io_dtype == KDA_BF16, p->dk, a, out, state_out, s));
}

kda_status kda_backward_after_prefill(const kda_problem* p, const void* q, const void* k, const void* v,
                                      const float* log_alpha, const float* beta, const void* g, const void* out,
                                      const void* d_out, const float* d_state, void* dq, void* dk, void* dv,
                                      float* dlog_alpha, float* dbeta, void* dg, float* d_state_in,
                                      void* workspace, size_t workspace_bytes, void* stream) {
    BackwardArgs a = {};
    bool work = false;
    const kda_status st = backward_args(p, q, k, v, log_alpha, beta, g, nullptr, out, true, d_out, d_state, dq,
                                        dk, dv, dlog_alpha, dbeta, dg, d_state_in, workspace, workspace_bytes, &a,
                                        &work);
    if (st != KDA_OK || !work) return st;
    return hip_status(launch_backward(p->io_dtype == KDA_BF16, p->dk, a, false, (hipStream_t)stream));
}

size_t kda_varlen_backward_workspace_size(const kda_problem* p, int64_t n_seq) {
    if (check_varlen(p, n_seq) != KDA_OK || n_seq == 0 || p->seqlen == 0) return 0;
    return backward_workspace_bytes(p->io_dtype == KDA_BF16, n_seq, p->seqlen, p->heads, p->dk, true);
}

kda_status kda_varlen_backward(const kda_problem* p, int64_t n_seq, const int32_t* cu_seqlens, const void* q,
                               const void* k, const void* v, const float* log_alpha, const float* beta, const void* g,
                               const float* state_in, const void* d_out, const float* d_state, void* dq, void* dk,
                               void* dv, float* dlog_alpha, float* dbeta, void* dg, float* d_state_in,
                               void* workspace, size_t workspace_bytes, void* stream) {
    kda_status st = check_varlen(p, n_seq);
    if (st != KDA_OK) return st;
    const bool tokens = p->seqlen > 0;
    if (!ok_beta(cu_seqlens, n_seq > 0) || !ok_ptr(q, tokens) || !ok_ptr(k, tokens) || !ok_ptr(v, tokens) ||
        !ok_ptr(log_alpha, tokens) || !ok_beta(beta, tokens) || !ok_ptr(g, tokens) || !ok_ptr(dq, tokens) ||
        !ok_ptr(dk, tokens) || !ok_ptr(dv, tokens) || !ok_ptr(dlog_alpha, tokens) || !ok_beta(dbeta, tokens) ||
        !ok_ptr(dg, tokens) || !ok_ptr(workspace, tokens && n_seq > 0) || !ok_opt_ptr(state_in) ||
        !ok_opt_ptr(d_out) || !ok_opt_ptr(d_state) || !ok_opt_ptr(d_state_in))
        return KDA_ERR_INVALID_ARGUMENT;
    if (workspace_bytes < kda_varlen_backward_workspace_size(p, n_seq)) return KDA_ERR_WORKSPACE_TOO_SMALL;
    if (n_seq == 0 || (!tokens && !d_state_in)) return KDA_OK;
    if ((st = device_ready()) != KDA_OK) return st;
    BackwardArgs a = {};
    a.q = q; a.k = k; a.v = v; a.log_alpha = log_alpha; a.beta = beta; a.g = g; a.state_in = state_in;
    a.d_out = d_out; a.d_state = d_state;
    a.dq = dq; a.dk = dk; a.dv = dv; a.dlog_alpha = dlog_alpha; a.dbeta = dbeta; a.dg = dg;
    a.d_state_in = d_state_in;
    a.ws = static_cast<char*>(workspace);
    a.B = n_seq; a.T = p->seqlen; a.H = p->heads; a.NC = 0; a.floor_ = p->log_alpha_min;
    // with no tokens every sequence is empty: the uniform path (no chunks,
    // no workspace) passes each sequence's state gradient through
    if (tokens) a.cu_seqlens = cu_seqlens;
    return hip_status(launch_backward(p->io_dtype == KDA_BF16, p->dk, a, true, (hipStream_t)stream));
}

kda_status kda_varlen_prefill_for_backward(const kda_problem* p, int64_t n_seq, const int32_t* cu_seqlens,
                                           const void* q, const void* k, const void* v, const float* log_alpha,
                                           const float* beta, const void* g, const float* state_in, void* out,
                                           float* state_out, void* workspace, size_t workspace_bytes,
                                           void* stream) {
    kda_status st = check_varlen(p, n_seq);
    if (st != KDA_OK) return st;
    const bool tokens = p->seqlen > 0;
    if (!ok_beta(cu_seqlens, n_seq > 0) || !ok_ptr(q, tokens) || !ok_ptr(k, tokens) || !ok_ptr(v, tokens) ||
        !ok_ptr(log_alpha, tokens) || !ok_beta(beta, tokens) || !ok_ptr(g, tokens) || !ok_ptr(out, tokens) ||
        !ok_ptr(workspace, tokens && n_seq > 0) || !ok_opt_ptr(state_in) || !ok_opt_ptr(state_out))
        return KDA_ERR_INVALID_ARGUMENT;
    if (workspace_bytes < kda_varlen_backward_workspace_size(p, n_seq)) return KDA_ERR_WORKSPACE_TOO_SMALL;
    if (n_seq == 0 || (!tokens && !state_out)) return KDA_OK;
    if ((st = device_ready()) != KDA_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    if (!tokens) {   // every sequence empty: its state passes through
        kda_problem each = *p;
        each.batch = n_seq;
        return copy_state(&each, state_in, state_out, s);
    }
    BackwardArgs a = {};
    a.q = q; a.k = k; a.v = v; a.log_alpha = log_alpha; a.beta = beta; a.g = g; a.state_in = state_in;
    a.ws = static_cast<char*>(workspace);
    a.cu_seqlens = cu_seqlens;
    a.B = n_seq; a.T = p->seqlen; a.H = p->heads; a.NC = 0; a.floor_ = p->log_alpha_min;
    return hip_status(launch_backward_forward(p->io_dtype == KDA_BF16, p->dk, a, out, state_out, s));
}

kda_status kda_varlen_backward_after_prefill(const kda_problem* p, int64_t n_seq, const int32_t* cu_seqlens,
                                             const void* q, const void* k, const void* v, const float* log_alpha,
                                             const float* beta, const void* g, const void* out, const void* d_out,
                                             const float* d_state, void* dq, void* dk, void* dv, float* dlog_alpha,
                                             float* dbeta, void* dg, float* d_state_in, void* workspace,
                                             size_t workspace_bytes, void* stream) {
    kda_status st = check_varlen(p, n_seq);
    if (st != KDA_OK) return st;
    const bool tokens = p->seqlen > 0;
    if (!ok_beta(cu_seqlens, n_seq > 0) || !ok_ptr(q, tokens) || !ok_ptr(k, tokens) || !ok_ptr(v, tokens) ||
        !ok_ptr(log_alpha, tokens) || !ok_beta(beta, tokens) || !ok_ptr(g, tokens) || !ok_ptr(out, tokens) ||
        !ok_ptr(dq, tokens) || !ok_ptr(dk, tokens) || !ok_ptr(dv, tokens) || !ok_ptr(dlog_alpha, tokens) ||
        !ok_beta(dbeta, tokens) || !ok_ptr(dg, tokens) || !ok_ptr(workspace, tokens && n_seq > 0) ||
        !ok_opt_ptr(d_out) || !ok_opt_ptr(d_state) || !ok_opt_ptr(d_state_in))
        return KDA_ERR_INVALID_ARGUMENT;
    if (workspace_bytes < kda_varlen_backward_workspace_size(p, n_seq)) return KDA_ERR_WORKSPACE_TOO_SMALL;
    if (n_seq == 0 || (!tokens && !d_state_in)) return KDA_OK;
    if ((st = device_ready()) != KDA_OK) return st;
    BackwardArgs a = {};
    a.q = q; a.k = k; a.v = v; a.log_alpha = log_alpha; a.beta = beta; a.g = g;
    a.d_out = d_out; a.d_state = d_state;
    a.dq = dq; a.dk = dk; a.dv = dv; a.dlog_alpha = dlog_alpha; a.dbeta = dbeta; a.dg = dg;
    a.d_state_in = d_state_in;
    a.out = out;
    a.ws = static_cast<char*>(workspace);
    a.B = n_seq; a.T = p->seqlen; a.H = p->heads; a.NC = 0; a.floor_ = p->log_alpha_min;
    if (tokens) a.cu_seqlens = cu_seqlens;   // else the uniform path passes the state gradients through
    return hip_status(launch_backward(p->io_dtype == KDA_BF16, p->dk, a, false, (hipStream_t)stream));
}

size_t kda_pipelined_workspace_size(const kda_problem* p, int32_t range_chunks) {
    if (check_problem(p) != KDA_OK || range_chunks < 1) return 0;
    const int64_t rc = range_of(p, range_chunks);
    const int nbuf = n_chunks(p) > rc ? 2 : 1;
    return state_bytes_of(p) + (size_t)nbuf * range_card_bytes(p, rc);
}

kda_status kda_prefill_pipelined(const kda_problem* p, const void* q, const void* k, const void* v,
                                 const float* log_alpha, const float* beta, const void* g, const float* state_in,
                                 void* out, float* state_out, int32_t range_chunks, void* workspace,
                                 size_t workspace_bytes, void* stream, void* aux_stream) {
    kda_status st = check_problem(p);
    if (st != KDA_OK) return st;
    if (range_chunks < 1) return KDA_ERR_INVALID_ARGUMENT;
    const bool tokens = p->batch > 0 && p->seqlen > 0;
    if (!ok_ptr(q, tokens) || !ok_ptr(k, tokens) || !ok_ptr(v, tokens) || !ok_ptr(log_alpha, tokens) ||
        !ok_beta(beta, tokens) || !ok_ptr(g, tokens) || !ok_ptr(out, tokens) || !ok_ptr(workspace, tokens) ||
        !ok_opt_ptr(state_in) || !ok_opt_ptr(state_out))
        return KDA_ERR_INVALID_ARGUMENT;
    if (workspace_bytes < kda_pipelined_workspace_size(p, range_chunks)) return KDA_ERR_WORKSPACE_TOO_SMALL;
    if (p->batch == 0 || (!tokens && !state_out)) return KDA_OK;
    hipStream_t s = (hipStream_t)stream, aux = (hipStream_t)aux_stream;
    const bool bf16 = p->io_dtype == KDA_BF16;
    const int64_t NC = n_chunks(p);
    if ((st = device_ready()) != KDA_OK) return st;
    if (NC == 0) return copy_state(p, state_in, state_out, s);
    const int64_t rc = range_of(p, range_chunks);
    float* carry = state_out ? state_out : static_cast<float*>(workspace);
    char* cards[2] = {static_cast<char*>(workspace) + state_bytes_of(p), nullptr};
    cards[1] = cards[0] + range_card_bytes(p, rc);
    auto range = [&](int64_t c0) {
        const int64_t c1 = c0 + rc < NC ? c0 + rc : NC;
        RangeLaunch r = range_launch(p, q, k, v, log_alpha, beta, g, out, cards[(c0 / rc) & 1], c0, c1);
        r.sa.state_in = c0 == 0 ? state_in : carry;
        r.sa.state_out = (c1 == NC && !state_out) ? nullptr : carry;
        return r;
    };
    if (rc == NC) {   // one range: nothing to overlap
        const RangeLaunch r = range(0);
        if (launch_prepare(bf16, p->dk, r.pa, s) != hipSuccess) return KDA_ERR_HIP;
        return hip_status(launch_scan(bf16, p->dk, false, r.sa, s));
    }
    // Events: the caller's prior work on `stream` (start), each card buffer
    // filled (prepared[b]) and drained (scanned[b]), and the aux stream's end
    // (joined), which `stream` waits on before returning, also on failure, so
    // nothing of this call runs on aux after the caller's next work on `stream`.
    enum { kStart, kPrep0, kPrep1, kScan0, kScan1, kJoin, kEvents };
    hipEvent_t ev[kEvents] = {};
    for (int i = 0; i < kEvents; ++i)
        if (hipEventCreateWithFlags(&ev[i], hipEventDisableTiming) != hipSuccess) {
            for (int j = 0; j < i; ++j) hipEventDestroy(ev[j]);
            return KDA_ERR_HIP;
        }
    bool ok = hipEventRecord(ev[kStart], s) == hipSuccess && hipStreamWaitEvent(aux, ev[kStart], 0) == hipSuccess;
    for (int64_t c0 = 0, i = 0; ok && c0 < NC; c0 += rc, ++i) {
        const int b = (int)(i & 1);
        const RangeLaunch r = range(c0);
        // range i's prepare on aux, once the scan of range i - 2 (same buffer) is done
        ok = (i < 2 || hipStreamWaitEvent(aux, ev[kScan0 + b], 0) == hipSuccess) &&
             launch_prepare(bf16, p->dk, r.pa, aux) == hipSuccess && hipEventRecord(ev[kPrep0 + b], aux) == hipSuccess &&
             hipStreamWaitEvent(s, ev[kPrep0 + b], 0) == hipSuccess &&
             launch_scan(bf16, p->dk, false, r.sa, s) == hipSuccess && hipEventRecord(ev[kScan0 + b], s) == hipSuccess;
    }
    const bool joined = hipEventRecord(ev[kJoin], aux) == hipSuccess && hipStreamWaitEvent(s, ev[kJoin], 0) == hipSuccess;
    for (int i = 0; i < kEvents; ++i) hipEventDestroy(ev[i]);
    return ok && joined ? KDA_OK : KDA_ERR_HIP;
}

kda_status kda_prefill_noalloc(const kda_problem* p, const void* q, const void* k, const void* v,
                               const float* log_alpha, const float* beta, const void* g, const float* state_in,
                               void* out, float* state_out, void* stream) {
    kda_status st = check_problem(p);
    if (st != KDA_OK) return st;
    const bool tokens = p->batch > 0 && p->seqlen > 0;
    if (!ok_ptr(q, tokens) || !ok_ptr(k, tokens) || !ok_ptr(v, tokens) || !ok_ptr(log_alpha, tokens) ||
        !ok_beta(beta, tokens) || !ok_ptr(g, tokens) || !ok_ptr(out, tokens) || !ok_opt_ptr(state_in) ||
        !ok_opt_ptr(state_out))
        return KDA_ERR_INVALID_ARGUMENT;
    if (p->batch == 0 || (!tokens && !state_out)) return KDA_OK;
    const bool bf16 = p->io_dtype == KDA_BF16;
    const int64_t NC = n_chunks(p);
    hipStream_t s = (hipStream_t)stream;
    if (NC == 0) {   // no tokens: state_out = state_in (or 0); no cards
        if ((st = device_ready()) != KDA_OK) return st;
        return copy_state(p, state_in, state_out, s);
    }
    const size_t BH = (size_t)p->batch * (size_t)p->heads;
    const size_t per_chunk = BH * card_bytes(bf16, p->dk);   // cards of one chunk index, all (row, head)
    // chunks per pass: all of them if their cards fit; otherwise as many as
    // fit beside the state carried between passes (in state_out when given,
    // else at the front of the scratch area)
    const size_t state_bytes = state_out ? 0 : (BH * (size_t)p->dk * (size_t)p->dv * 4 + 255) / 256 * 256;
    int64_t per_pass = (int64_t)(KDA_NOALLOC_SCRATCH_BYTES / per_chunk);
    size_t cards_off = 0;
    if (per_pass < NC) {
        if (state_bytes >= KDA_NOALLOC_SCRATCH_BYTES) return KDA_ERR_WORKSPACE_TOO_SMALL;
        per_pass = (int64_t)((KDA_NOALLOC_SCRATCH_BYTES - state_bytes) / per_chunk);
        cards_off = state_bytes;
    }
    if (per_pass < 1) return KDA_ERR_WORKSPACE_TOO_SMALL;
    if ((st = device_ready()) != KDA_OK) return st;
    void* base = nullptr;
    if ((st = scratch_address(&base)) != KDA_OK) return st;
    char* cards = static_cast<char*>(base) + cards_off;
    float* carry = state_out ? state_out : reinterpret_cast<float*>(base);
    for (int64_t c0 = 0; c0 < NC; c0 += per_pass) {
        const int64_t c1 = c0 + per_pass < NC ? c0 + per_pass : NC;
        RangeLaunch r = range_launch(p, q, k, v, log_alpha, beta, g, out, cards, c0, c1);
        r.sa.state_in = c0 == 0 ? state_in : carry;
        r.sa.state_out = (c1 == NC && !state_out) ? nullptr : carry;
        if (launch_prepare(bf16, p->dk, r.pa, s) != hipSuccess) return KDA_ERR_HIP;
        if (launch_scan(bf16, p->dk, false, r.sa, s) != hipSuccess) return KDA_ERR_HIP;
    }
    return KDA_OK;
}

}  // extern "C"
