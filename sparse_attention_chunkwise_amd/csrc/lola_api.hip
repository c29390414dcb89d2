// C ABI of liblola: argument checks, layouts and kernel launches.
// Every check happens on the host before anything is enqueued.
#include <dlfcn.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "lola_decode.h"
#include "lola_internal.h"
#include "lola_misc.h"
#include "lola_output.h"
#include "lola_decode_bf16.h"
#include "lola_prefill.h"
#include "lola_scan_split.h"

using namespace lola;

// Workspace of lola_prefill_chunk_noalloc: one array per GPU, held from the first
// use until the process ends.  In host code `scratch` names a host-side stand-in,
// not device memory: only the address hipGetSymbolAddress returns for the current
// device (kept in scratch_ptr) may be passed to kernels.  Every call on a GPU uses
// the same array and leaves its contents behind; the kernels clear what must start
// at zero (the prologue zeroes the split scan's exchange slots and counters).
constexpr size_t kNoallocScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices] = {};

// Device address of this GPU's `scratch` (looked up once per device, with the
// stream's device current).
lola_status noalloc_scratch(hipStream_t stream, void** out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return LOLA_ERR_HIP;
    if (stream) {
        int sdev = -1;
        if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return LOLA_ERR_HIP;
        if (sdev != dev) return LOLA_ERR_INVALID_ARG;  // the stream must belong to the current device
    }
    if (dev < 0 || dev >= kMaxDevices) return LOLA_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return LOLA_ERR_HIP;
        scratch_ptr[dev] = p;
    }
    *out = scratch_ptr[dev];
    return LOLA_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Host-side ranges for profilers: with LOLA_TRACE=1 in the environment every kernel
// launch is enclosed in a roctx range named after the kernel (rocprofv3 --marker-trace
// records them).  The roctx library is opened at the first launch and only then;
// without the variable, or without the library, a launch pays one branch.
struct Tracer {
    bool on = false;
    int (*push)(const char*) = nullptr;
    int (*pop)() = nullptr;
};
const Tracer& tracer()
{
    static const Tracer t = [] {
        Tracer r;
        const char* e = getenv("LOLA_TRACE");
        if (!e || strcmp(e, "1") != 0) return r;
        void* h = dlopen("librocprofiler-sdk-roctx.so.1", RTLD_NOW | RTLD_LOCAL);
        if (!h) h = dlopen("libroctx64.so.4", RTLD_NOW | RTLD_LOCAL);
        if (!h) return r;
        r.push = reinterpret_cast<int (*)(const char*)>(dlsym(h, "roctxRangePushA"));
        r.pop = reinterpret_cast<int (*)()>(dlsym(h, "roctxRangePop"));
        r.on = r.push && r.pop;
        return r;
    }();
    return t;
}
struct TraceRange {
    bool on;
    explicit TraceRange(const char* name) : on(tracer().on)
    {
        if (on) tracer().push(name);
    }
    ~TraceRange()
    {
        if (on) tracer().pop();
    }
};

lola_status make_dims(const lola_config* cfg, Dims* d)
{
    if (!cfg) return LOLA_ERR_INVALID_ARG;
    if (cfg->n_kv_heads < 1 || cfg->n_q_heads < 1 || cfg->head_dim < 1 || cfg->feat_half < 1 || cfg->window < 0 ||
        cfg->cache_cap < 0 || cfg->chunk < 1)
        return LOLA_ERR_INVALID_ARG;
    if (cfg->n_q_heads % cfg->n_kv_heads != 0) return LOLA_ERR_INVALID_ARG;
    if (cfg->n_q_heads / cfg->n_kv_heads > kMaxGroup) return LOLA_ERR_UNSUPPORTED;
    if (cfg->head_dim != 64 && cfg->head_dim != 128) return LOLA_ERR_UNSUPPORTED;
    if (cfg->feat_half != 32 && cfg->feat_half != 64) return LOLA_ERR_UNSUPPORTED;
    if (cfg->window > kMaxWindow || cfg->cache_cap > kMaxCache || cfg->chunk > kMaxChunk) return LOLA_ERR_UNSUPPORTED;
    if (cfg->io_dtype != LOLA_F32 && cfg->io_dtype != LOLA_BF16) return LOLA_ERR_UNSUPPORTED;
    if (!(cfg->softmax_scale == cfg->softmax_scale)) return LOLA_ERR_INVALID_ARG;  // NaN
    if (cfg->policy < LOLA_POLICY_SRE || cfg->policy > LOLA_POLICY_SOFTMAX_ERR) return LOLA_ERR_UNSUPPORTED;
    if (cfg->decode_mode != LOLA_DECODE_RESCORE && cfg->decode_mode != LOLA_DECODE_INCREMENTAL)
        return LOLA_ERR_UNSUPPORTED;
    if (cfg->decode_mode == LOLA_DECODE_INCREMENTAL && (cfg->io_dtype != LOLA_BF16 || cfg->policy != LOLA_POLICY_SRE))
        return LOLA_ERR_UNSUPPORTED;
    d->Hq = cfg->n_q_heads;
    d->Hkv = cfg->n_kv_heads;
    d->D = cfg->head_dim;
    d->Fh = cfg->feat_half;
    d->F = 2 * cfg->feat_half;
    d->w = cfg->window;
    d->C = cfg->cache_cap;
    d->L = cfg->chunk;
    d->G = cfg->n_q_heads / cfg->n_kv_heads;
    d->io = cfg->io_dtype;
    d->esize = cfg->io_dtype == LOLA_BF16 ? 2 : 4;
    d->tau = cfg->softmax_scale > 0.f ? cfg->softmax_scale : 1.0f / sqrtf((float)cfg->head_dim);
    d->policy = cfg->policy;
    d->inc = cfg->decode_mode == LOLA_DECODE_INCREMENTAL ? 1 : 0;
    return LOLA_OK;
}

uint64_t cfg_hash(const lola_config* c, int batch)
{
    uint64_t h = 1469598103934665603ull;
    auto mix = [&](uint32_t x) {
        for (int i = 0; i < 4; ++i) {
            h ^= (x >> (8 * i)) & 0xffu;
            h *= 1099511628211ull;
        }
    };
    uint32_t sc;
    memcpy(&sc, &c->softmax_scale, 4);
    mix((uint32_t)c->n_q_heads); mix((uint32_t)c->n_kv_heads); mix((uint32_t)c->head_dim);
    mix((uint32_t)c->feat_half); mix((uint32_t)c->window); mix((uint32_t)c->cache_cap);
    mix((uint32_t)c->chunk); mix((uint32_t)c->io_dtype); mix(sc); mix((uint32_t)batch);
    if (c->policy != 0) mix(0x9e3779b9u ^ (uint32_t)c->policy);
    if (c->decode_mode != 0) mix(0x85ebca6bu ^ (uint32_t)c->decode_mode);
    return h;
}

lola_status check_batch(int32_t batch, const Dims& d)
{
    if (batch < 1) return LOLA_ERR_INVALID_ARG;
    if ((int64_t)batch * d.Hkv > 65535) return LOLA_ERR_UNSUPPORTED;
    return LOLA_OK;
}

lola_status hip_status(hipError_t e) { return e == hipSuccess ? LOLA_OK : LOLA_ERR_HIP; }

template <typename K>
hipError_t allow_lds(K kernel, size_t bytes)
{
    return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)bytes);
}

hipError_t mark(void* const* events, int i, hipStream_t s)
{
    if (!events || !events[i]) return hipSuccess;
    return hipEventRecord((hipEvent_t)events[i], s);
}

// The split scan needs every block of a chain resident at once: a cooperative
// launch on a device that supports it, with the grid within the device's
// co-resident capacity.  LOLA_SCAN_SPLIT=0 in the environment selects the
// one-block-per-chain scan everywhere.
bool split_allowed()
{
    const char* e = getenv("LOLA_SCAN_SPLIT");
    return !(e && e[0] == '0');
}

template <typename K>
bool split_fits(K kernel, int blocks, size_t lds)
{
    int dev = 0, coop = 0, ncu = 0, per = 0;
    if (hipGetDevice(&dev) != hipSuccess) return false;
    if (hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev) != hipSuccess || !coop) return false;
    if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return false;
    if (allow_lds(kernel, lds) != hipSuccess) return false;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, reinterpret_cast<const void*>(kernel), kSplitThreads,
                                                     lds) != hipSuccess)
        return false;
    return (int64_t)per * ncu >= blocks;
}

template <int D, int F, typename T>
lola_status launch_prefill(Args& a, hipStream_t s, void* const* ev)
{
    const Dims& d = a.d;
    const int chains = a.B * d.Hkv;
    if (mark(ev, 0, s) != hipSuccess) return LOLA_ERR_HIP;
    // the scan variant decides which phi rows the prologue writes: the split scan
    // (bf16 io) reads the bf16 hi/lo rows only
    int pu = 0;
    size_t split_lds = 0;
    if constexpr (sizeof(T) == 2) {
        split_lds = split_smem<F>().total;
        // as many candidate groups per column slice (4, 2, then 1) as the device holds at
        // once; the scoring policies other than the SRE run in the one-workgroup scan
        if (split_allowed() && d.policy == LOLA_POLICY_SRE)
            for (int g : {4, 2, 1})
                if (split_fits(scan_split_kernel<D, F>, split_blocks(D, chains, g), split_lds)) {
                    pu = g;
                    break;
                }
    }
    const bool split = pu > 0;
    dim3 gp((a.wl.X + d.C + 63) / 64, chains);
    {
        TraceRange tr("lola::prologue");
        if constexpr (sizeof(T) == 2)
            hipLaunchKernelGGL((prologue_bf16_kernel<D, F / 2>), gp, dim3(256), 0, s, a, split ? 0 : 1);
        else
            hipLaunchKernelGGL((prologue_kernel<D, F / 2, T>), gp, dim3(256), 0, s, a);
    }
    if (hipGetLastError() != hipSuccess || mark(ev, 1, s) != hipSuccess) return LOLA_ERR_HIP;
    if constexpr (sizeof(T) == 2) {
        if (split) {
            TraceRange tr("lola::scan_split");
            if (allow_lds(scan_split_kernel<D, F>, split_lds) != hipSuccess) return LOLA_ERR_HIP;
            void* params[] = {&a};
            if (hipLaunchCooperativeKernel(reinterpret_cast<const void*>(scan_split_kernel<D, F>),
                                           dim3(split_blocks(D, chains, pu)), dim3(kSplitThreads), params,
                                           (unsigned)split_lds, s) != hipSuccess)
                return LOLA_ERR_HIP;
        }
    }
    if (!split) {
        TraceRange tr("lola::scan");
        const size_t scan_lds = scan_smem(D, F, d.C, d.L, sizeof(T)).total;
        if (allow_lds(scan_kernel<D, F, T>, scan_lds) != hipSuccess) return LOLA_ERR_HIP;
        hipLaunchKernelGGL((scan_kernel<D, F, T>), dim3(chains), dim3(scan_threads(D)), scan_lds, s, a);
    }
    if (hipGetLastError() != hipSuccess || mark(ev, 2, s) != hipSuccess) return LOLA_ERR_HIP;
    {
        TraceRange tr("lola::output");
        if constexpr (sizeof(T) == 2) {
            const int wpi = (d.G * d.L + kOutRows - 1) / kOutRows;
            const size_t olds = out_smem<D, F>(d.C).total;
            if (allow_lds(output_kernel_bf16<D, F>, olds) != hipSuccess) return LOLA_ERR_HIP;
            hipLaunchKernelGGL((output_kernel_bf16<D, F>), dim3(a.NI * wpi, chains), dim3(kOutThreads), olds, s, a);
        } else {
            const int wpi = (d.G * d.L + 63) / 64;
            hipLaunchKernelGGL((output_kernel<D, F, T>), dim3(a.NI * wpi, chains), dim3(256), 0, s, a);
        }
    }
    if (hipGetLastError() != hipSuccess || mark(ev, 3, s) != hipSuccess) return LOLA_ERR_HIP;
    return LOLA_OK;
}

template <int D, int F, typename T>
lola_status launch_decode(Args& a, hipStream_t s)
{
    TraceRange tr("lola::decode");
    if constexpr (sizeof(T) == 2) {
        const size_t lds = dec_smem<D, F>(a.d.C).total;
        if (a.d.inc) {
            if (allow_lds(decode_kernel_bf16<D, F, true>, lds) != hipSuccess) return LOLA_ERR_HIP;
            hipLaunchKernelGGL((decode_kernel_bf16<D, F, true>), dim3(a.B * a.d.Hkv), dim3(kDecThreads), lds, s, a);
            return hip_status(hipGetLastError());
        }
        if (allow_lds(decode_kernel_bf16<D, F, false>, lds) != hipSuccess) return LOLA_ERR_HIP;
        hipLaunchKernelGGL((decode_kernel_bf16<D, F, false>), dim3(a.B * a.d.Hkv), dim3(kDecThreads), lds, s, a);
    } else {
        const size_t lds = decode_smem(D, F, a.d.G, a.d.C).total;
        if (allow_lds(decode_kernel<D, F, T>, lds) != hipSuccess) return LOLA_ERR_HIP;
        hipLaunchKernelGGL((decode_kernel<D, F, T>), dim3(a.B * a.d.Hkv), dim3(256), lds, s, a);
    }
    return hip_status(hipGetLastError());
}

#define LOLA_DISPATCH(FN, ...)                                                           \
    do {                                                                                 \
        const Dims& dd = a.d;                                                            \
        if (dd.io == LOLA_F32) {                                                         \
            if (dd.D == 64 && dd.F == 64) return FN<64, 64, float>(__VA_ARGS__);         \
            if (dd.D == 64 && dd.F == 128) return FN<64, 128, float>(__VA_ARGS__);       \
            if (dd.D == 128 && dd.F == 64) return FN<128, 64, float>(__VA_ARGS__);       \
            if (dd.D == 128 && dd.F == 128) return FN<128, 128, float>(__VA_ARGS__);     \
        } else {                                                                         \
            if (dd.D == 64 && dd.F == 64) return FN<64, 64, bf16>(__VA_ARGS__);          \
            if (dd.D == 64 && dd.F == 128) return FN<64, 128, bf16>(__VA_ARGS__);        \
            if (dd.D == 128 && dd.F == 64) return FN<128, 64, bf16>(__VA_ARGS__);        \
            if (dd.D == 128 && dd.F == 128) return FN<128, 128, bf16>(__VA_ARGS__);      \
        }                                                                                \
        return LOLA_ERR_UNSUPPORTED;                                                     \
    } while (0)

lola_status dispatch_prefill(Args& a, hipStream_t s, void* const* ev) { LOLA_DISPATCH(launch_prefill, a, s, ev); }
lola_status dispatch_decode(Args& a, hipStream_t s) { LOLA_DISPATCH(launch_decode, a, s); }

Args base_args(const lola_config* cfg, const Dims& d, int B, void* state)
{
    Args a;
    memset(&a, 0, sizeof(a));
    a.d = d;
    a.B = B;
    a.hash = cfg_hash(cfg, B);
    a.state = (unsigned char*)state;
    a.sl = state_layout(d, B);
    return a;
}

// one prefill call: seqn = per-sequence token counts on the device, or null (n_tokens for all)
lola_status prefill_impl(const lola_config* cfg, void* state, int32_t batch, int32_t n_tokens, const int32_t* seqn,
                         const void* q, const void* k, const void* v, void* out, void* workspace,
                         size_t workspace_bytes, void* stream, void* const* events)
{
    Dims d;
    lola_status st = make_dims(cfg, &d);
    if (st != LOLA_OK) return st;
    if ((st = check_batch(batch, d)) != LOLA_OK) return st;
    if (n_tokens < 1) return LOLA_ERR_INVALID_ARG;
    if (!state || !q || !k || !v || !out || !workspace) return LOLA_ERR_INVALID_ARG;
    if (!aligned16(state) || !aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) ||
        !aligned16(workspace))
        return LOLA_ERR_INVALID_ARG;
    Args a = base_args(cfg, d, batch, state);
    a.n = n_tokens;
    a.wl = ws_layout(d, batch, n_tokens);
    a.NI = a.wl.NI;
    if (workspace_bytes < a.wl.total) return LOLA_ERR_WORKSPACE;
    if ((int64_t)a.NI * ((d.G * d.L + 63) / 64) > 0x7fffffff) return LOLA_ERR_UNSUPPORTED;  // grid x
    a.ws = (unsigned char*)workspace;
    a.q = q;
    a.k = k;
    a.v = v;
    a.out = out;
    a.seqn = seqn;
    return dispatch_prefill(a, (hipStream_t)stream, events);
}

}  // namespace

extern "C" {

size_t lola_state_bytes(const lola_config* cfg, int32_t batch)
{
    Dims d;
    if (make_dims(cfg, &d) != LOLA_OK || check_batch(batch, d) != LOLA_OK) return 0;
    return state_layout(d, batch).total;
}

size_t lola_prefill_workspace_bytes(const lola_config* cfg, int32_t batch, int32_t max_tokens)
{
    Dims d;
    if (make_dims(cfg, &d) != LOLA_OK || check_batch(batch, d) != LOLA_OK || max_tokens < 1) return 0;
    return ws_layout(d, batch, max_tokens).total;
}

lola_status lola_init_state(const lola_config* cfg, int32_t batch, const float* W, void* state, void* stream)
{
    Dims d;
    lola_status st = make_dims(cfg, &d);
    if (st != LOLA_OK) return st;
    if ((st = check_batch(batch, d)) != LOLA_OK) return st;
    if (!W || !state || !aligned16(W) || !aligned16(state)) return LOLA_ERR_INVALID_ARG;
    Args a = base_args(cfg, d, batch, state);
    hipLaunchKernelGGL(init_kernel, dim3(batch * d.Hkv + 1), dim3(256), 0, (hipStream_t)stream, a, W,
                       cfg_hash(cfg, batch));
    return hip_status(hipGetLastError());
}

lola_status lola_prefill_chunk(const lola_config* cfg, void* state, int32_t batch, int32_t n_tokens, const void* q,
                               const void* k, const void* v, void* out, void* workspace, size_t workspace_bytes,
                               void* stream)
{
    return lola_prefill_chunk_timed(cfg, state, batch, n_tokens, q, k, v, out, workspace, workspace_bytes, stream,
                                    nullptr);
}

lola_status lola_prefill_chunk_timed(const lola_config* cfg, void* state, int32_t batch, int32_t n_tokens,
                                     const void* q, const void* k, const void* v, void* out, void* workspace,
                                     size_t workspace_bytes, void* stream, void* const* events)
{
    return prefill_impl(cfg, state, batch, n_tokens, nullptr, q, k, v, out, workspace, workspace_bytes, stream,
                        events);
}

lola_status lola_prefill_chunk_noalloc(const lola_config* cfg, void* state, int32_t batch, int32_t n_tokens,
                                       const void* q, const void* k, const void* v, void* out, void* stream)
{
    Dims d;
    lola_status st = make_dims(cfg, &d);
    if (st != LOLA_OK) return st;
    if ((st = check_batch(batch, d)) != LOLA_OK) return st;
    if (n_tokens < 1) return LOLA_ERR_INVALID_ARG;
    if (ws_layout(d, batch, n_tokens).total > kNoallocScratchBytes) return LOLA_ERR_WORKSPACE;
    void* ws = nullptr;
    if ((st = noalloc_scratch((hipStream_t)stream, &ws)) != LOLA_OK) return st;
    return prefill_impl(cfg, state, batch, n_tokens, nullptr, q, k, v, out, ws, kNoallocScratchBytes, stream,
                        nullptr);
}

lola_status lola_prefill_ragged(const lola_config* cfg, void* state, int32_t batch, int32_t max_tokens,
                                const int32_t* n_tokens, const void* q, const void* k, const void* v, void* out,
                                void* workspace, size_t workspace_bytes, void* stream)
{
    if (!n_tokens || ((uintptr_t)n_tokens & 3u)) return LOLA_ERR_INVALID_ARG;
    return prefill_impl(cfg, state, batch, max_tokens, n_tokens, q, k, v, out, workspace, workspace_bytes, stream,
                        nullptr);
}


lola_status lola_decode_step(const lola_config* cfg, void* state, int32_t batch, const void* q, const void* k,
                             const void* v, void* out, void* stream)
{
    Dims d;
    lola_status st = make_dims(cfg, &d);
    if (st != LOLA_OK) return st;
    if ((st = check_batch(batch, d)) != LOLA_OK) return st;
    if (!state || !q || !k || !v || !out) return LOLA_ERR_INVALID_ARG;
    if (!aligned16(state) || !aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
        return LOLA_ERR_INVALID_ARG;
    if (d.policy != LOLA_POLICY_SRE) return LOLA_ERR_UNSUPPORTED;  // lola_prefill_chunk(n_tokens = 1) runs it
    Args a = base_args(cfg, d, batch, state);
    a.n = 1;
    a.NI = 1;
    a.q = q;
    a.k = k;
    a.v = v;
    a.out = out;
    return dispatch_decode(a, (hipStream_t)stream);
}

lola_status lola_read_cache(const lola_config* cfg, const void* state, int32_t batch, int32_t* count, int64_t* pos,
                            void* k_out, void* v_out, float* H_out, float* s_out, int64_t* tokens_seen, void* stream)
{
    Dims d;
    lola_status st = make_dims(cfg, &d);
    if (st != LOLA_OK) return st;
    if ((st = check_batch(batch, d)) != LOLA_OK) return st;
    if (!state || !aligned16(state)) return LOLA_ERR_INVALID_ARG;
    const void* outs[] = {count, pos, k_out, v_out, H_out, s_out, tokens_seen};
    for (const void* p : outs)
        if (p && ((uintptr_t)p & 7u)) return LOLA_ERR_INVALID_ARG;
    Args a = base_args(cfg, d, batch, const_cast<void*>(state));
    hipStream_t s = (hipStream_t)stream;
    if (d.io == LOLA_F32)
        hipLaunchKernelGGL(read_cache_kernel<float>, dim3(batch * d.Hkv), dim3(256), 0, s, a, count, pos,
                           (float*)k_out, (float*)v_out, H_out, s_out, tokens_seen);
    else
        hipLaunchKernelGGL(read_cache_kernel<bf16>, dim3(batch * d.Hkv), dim3(256), 0, s, a, count, pos,
                           (bf16*)k_out, (bf16*)v_out, H_out, s_out, tokens_seen);
    return hip_status(hipGetLastError());
}

lola_status lola_check_state(const lola_config* cfg, const void* state, int32_t batch, void* stream)
{
    Dims d;
    lola_status st = make_dims(cfg, &d);
    if (st != LOLA_OK) return st;
    if ((st = check_batch(batch, d)) != LOLA_OK) return st;
    if (!state) return LOLA_ERR_INVALID_ARG;
    if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return LOLA_ERR_HIP;
    StateHeader h;
    if (hipMemcpy(&h, state, sizeof(h), hipMemcpyDeviceToHost) != hipSuccess) return LOLA_ERR_HIP;
    if (h.magic != kMagic || h.version != kVersion || h.cfg_hash != cfg_hash(cfg, batch) || h.batch != batch ||
        h.fault != 0)
        return LOLA_ERR_BAD_STATE;
    return LOLA_OK;
}

const char* lola_status_string(lola_status status)
{
    switch (status) {
    case LOLA_OK: return "ok";
    case LOLA_ERR_INVALID_ARG: return "invalid argument (null or misaligned pointer, bad count or size)";
    case LOLA_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case LOLA_ERR_BAD_STATE: return "state header does not match the configuration";
    case LOLA_ERR_WORKSPACE: return "workspace too small";
    case LOLA_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

}  // extern "C"
