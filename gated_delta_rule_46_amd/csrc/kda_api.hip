// kda_api.hip -- the C ABI declared in include/kda.h: argument validation,
// workspace sizing and launch planning.  Every check runs on the host before
// the first launch, so a call either enqueues all of its work or none of it.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "kda.h"
#include "kda_internal.h"
#include "kda_ops.h"

namespace {

thread_local std::string g_last_error;

int fail(int status, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return status;
}

int ok() {
    g_last_error.clear();
    return KDA_OK;
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Shared checks of the problem description; `decode` selects the decode
// kernel's shape set instead of the chunk engine's.
int check_config(const kda_config *cfg, bool decode = false) {
    if (!cfg) return fail(KDA_ERR_ARG, "cfg is NULL");
    if (cfg->num_heads <= 0) return fail(KDA_ERR_ARG, "num_heads must be positive (got %d)", cfg->num_heads);
    if (cfg->io_dtype != KDA_DTYPE_F32 && cfg->io_dtype != KDA_DTYPE_BF16)
        return fail(KDA_ERR_ARG, "io_dtype must be KDA_DTYPE_F32 or KDA_DTYPE_BF16 (got %d)", cfg->io_dtype);
    if (cfg->qk_l2norm != 0 && cfg->qk_l2norm != 1)
        return fail(KDA_ERR_ARG, "qk_l2norm must be 0 or 1 (got %d)", cfg->qk_l2norm);
    if (!std::isfinite(cfg->scale)) return fail(KDA_ERR_ARG, "scale must be finite");
    if (cfg->chunk != kda::kChunk)
        return fail(KDA_ERR_UNSUPPORTED, "chunk must be %d (got %d)", kda::kChunk, cfg->chunk);
    const bool bf = cfg->io_dtype == KDA_DTYPE_BF16;
    if (decode) {
        if (!kda::decode_supported(cfg->dk, cfg->dv))
            return fail(KDA_ERR_UNSUPPORTED, "unsupported head dims dk=%d dv=%d for decode",
                        cfg->dk, cfg->dv);
        return KDA_OK;
    }
    if (!kda::engine_supported(bf, cfg->dk, cfg->dv, 64))
        return fail(KDA_ERR_UNSUPPORTED, "unsupported head dims dk=%d dv=%d for %s I/O", cfg->dk,
                    cfg->dv, bf ? "bf16" : "fp32");
    return KDA_OK;
}

int check_tensor(const void *p, const char *name, bool required, size_t align = 16) {
    if (!p) return required ? fail(KDA_ERR_ARG, "%s is NULL", name) : KDA_OK;
    if (!aligned(p, align)) return fail(KDA_ERR_ALIGN, "%s is not %zu-byte aligned", name, align);
    return KDA_OK;
}

int check_ckpt_interval(int32_t interval) {
    if (interval <= 0 || interval % kda::kChunk != 0)
        return fail(KDA_ERR_ARG, "checkpoint interval must be a positive multiple of %d (got %d)",
                    kda::kChunk, interval);
    return KDA_OK;
}

int launched(hipError_t e, const char *what) {
    if (e != hipSuccess) return fail(KDA_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

#define KDA_TRY(x)                 \
    do {                           \
        const int _st = (x);       \
        if (_st != KDA_OK) return _st; \
    } while (0)

size_t round256(size_t b) { return (b + 255) / 256 * 256; }

size_t prefill_ws_bytes(int32_t N) { return round256((size_t)(N > 0 ? N : 1) * sizeof(int32_t)); }

// Compute units of the current device (queried once per device).
int device_cus() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
        v = 256;
    cache[dev].store(v, std::memory_order_relaxed);
    return v;
}

// One long sequence on too few workgroups runs faster as segments: packages
// of every segment in parallel, a scan over them, then the outputs fixed up
// from each segment's incoming state (the segment path), all inside the
// caller's workspace.
constexpr int64_t kMinSplit = 512;   // shortest segment worth a workgroup of its own

// Chunks of rows the internal split keeps of each segment's fix-up operator.
constexpr int kSplitFixopChunks = 6;

struct SplitPlan {
    int nseg = 0;
    int64_t L = 0, rows = 0;
    size_t off_M = 0, off_D = 0, off_Sin = 0, off_Sfin = 0, off_subD = 0, off_bounds = 0,
           off_X = 0, off_Xlen = 0, off_route = 0, off_Pi = 0, off_flags = 0, bytes = 0;
    bool fixop = false;
};

bool plan_split(const kda_config *cfg, int64_t T, int32_t N, const kda_ckpt *ckpt, SplitPlan *p,
                bool fixop = true) {
    if (N != 1 || T < 2 * kMinSplit) return false;
    if (ckpt && ckpt->offsets) return false;   // a device-side first rung row is not known here
    if (ckpt && (ckpt->interval <= 0 || ckpt->interval % kda::kChunk != 0)) return false;
    const bool bf = cfg->io_dtype == KDA_DTYPE_BF16;
    const int H = cfg->num_heads;
    if (!kda::engine_supported(bf, cfg->dk, cfg->dv, 64)) return false;
    const int nb = kda::engine_pick_nb(bf, cfg->dk, cfg->dv, H, kda::kModePrefill);
    const int cus = device_cus();
    if ((int64_t)H * (cfg->dv / nb) >= cus) return false;
    int64_t nseg = (cus + H - 1) / H;
    nseg = std::min<int64_t>(nseg, T / kMinSplit);
    if (nseg < 2) return false;
    const int64_t L = (T + nseg - 1) / nseg;
    p->L = (L + kda::kChunk - 1) / kda::kChunk * kda::kChunk;
    p->nseg = (int)((T + p->L - 1) / p->L);
    if (p->nseg < 2) return false;
    p->rows = ckpt ? T / ckpt->interval : 0;
    const size_t mm = (size_t)H * cfg->dk * cfg->dk * sizeof(float);
    const size_t dd = (size_t)H * cfg->dk * cfg->dv * sizeof(float);
    size_t at = 0;
    auto take = [&](size_t b) { const size_t o = at; at += round256(b); return o; };
    p->off_M = take(mm * p->nseg);
    p->off_D = take(dd * p->nseg);
    p->off_Sin = take(dd * p->nseg);
    p->off_Sfin = take(dd);
    p->off_subD = take(dd * (size_t)p->rows);
    p->off_bounds = take(sizeof(int64_t) * (size_t)(p->nseg + 1));
    p->off_flags = take(kda::sequential_workspace(H, p->nseg));   // the scan's zero tests of M
    // the fix-up operator (the chunked engine's shapes only)
    p->fixop = fixop && !kda::recurrent_supported(bf, cfg->dk, cfg->dv);
    if (p->fixop) {
        const size_t io = bf ? 2 : 4;
        p->off_X = take((size_t)p->nseg * kSplitFixopChunks * kda::kChunk * H * cfg->dk * io);
        p->off_Xlen = take((size_t)p->nseg * H * (cfg->dk / 64) * sizeof(int32_t));
        p->off_route = take((size_t)p->nseg * H * sizeof(int32_t));
        if (p->rows) p->off_Pi = take(mm * p->nseg);   // Pi at the rungs' interval
    }
    p->bytes = at;
    return true;
}

int prefill_split(const SplitPlan &p, const kda_config *cfg, const void *q, const void *k,
                  const void *v, const float *g, const float *beta, int64_t T, const float *S0,
                  float *S_final, void *o, const kda_ckpt *ckpt, void *ws, hipStream_t s) {
    unsigned char *w = (unsigned char *)ws;
    float *M = (float *)(w + p.off_M), *D = (float *)(w + p.off_D);
    float *S_in = (float *)(w + p.off_Sin);
    float *S_fin = S_final ? S_final : (float *)(w + p.off_Sfin);
    float *sub_D = p.rows ? (float *)(w + p.off_subD) : nullptr;
    int64_t *bounds = (int64_t *)(w + p.off_bounds);
    const bool bf = cfg->io_dtype == KDA_DTYPE_BF16;
    const int H = cfg->num_heads, dk = cfg->dk, dv = cfg->dv;
    hipError_t e = kda::launch_even_bounds(bounds, p.nseg, p.L, T, s);
    if (e != hipSuccess) return launched(e, "prefill split (bounds)");
    const int nb = kda::engine_pick_nb(bf, dk, dv, (int64_t)p.nseg * H, kda::kModePackage);
    kda::EngineArgs a{};
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.o = o;
    a.bounds = bounds; a.order = nullptr; a.n_units = p.nseg; a.H = H;
    a.S_init = nullptr; a.S_out = D; a.M_out = M;
    a.interval = p.rows ? ckpt->interval : 0;
    a.ckpt_off = nullptr; a.ckpt_S = sub_D; a.ckpt_M = nullptr;   // rungs come from the fix-up
    a.scale = cfg->scale; a.l2norm = cfg->qk_l2norm;
    a.ncb = dv / nb;
    a.ncb_m = dk / std::min(nb, dk);   // M has dk columns
    if (p.fixop) {   // the M blocks keep the fix-up operator of their first chunks
        a.X = w + p.off_X; a.X_len = (int32_t *)(w + p.off_Xlen); a.X_chunks = kSplitFixopChunks;
        if (p.rows) {
            a.X_Pi = (float *)(w + p.off_Pi); a.X_interval = ckpt->interval;
        }
    }
    if ((e = kda::launch_engine(kda::kModePackageVM, bf, dk, dv, nb, a, s)) != hipSuccess)
        return launched(e, "prefill split (package)");
    if ((e = kda::launch_scan_sequential(dk, dv, H, p.nseg, M, D, S0, S_in, S_fin,
                                         (int *)(w + p.off_flags), s)) != hipSuccess)
        return launched(e, "prefill split (scan)");
    kda::EngineArgs f{};
    f.q = q; f.k = k; f.v = nullptr; f.g = g; f.beta = beta; f.o = o;
    f.bounds = bounds; f.order = nullptr; f.n_units = p.nseg; f.H = H;
    f.S_init = S_in; f.scale = cfg->scale; f.l2norm = cfg->qk_l2norm;
    if (p.rows) {   // the fix-up writes the rungs: its propagated state plus sub_D
        f.interval = ckpt->interval; f.ckpt_S = ckpt->states; f.ckpt_in = sub_D;
    }
    const int nbf = kda::engine_pick_nb(bf, dk, dv, (int64_t)p.nseg * H, kda::kModeFixup);
    f.ncb = dv / nbf;
    if (p.fixop) {   // the units the operator covers, then the recurrence for the rest
        kda::EngineArgs x = f;
        x.X = a.X; x.X_len = a.X_len; x.X_chunks = a.X_chunks;
        x.X_Pi = a.X_Pi; x.X_interval = a.X_interval;
        x.X_route = (int32_t *)(w + p.off_route);
        if ((e = kda::launch_engine(kda::kModeFixOp, bf, dk, dv, nbf, x, s)) != hipSuccess)
            return launched(e, "prefill split (fix-up operator)");
        f.X_route = x.X_route;
    }
    return launched(kda::launch_engine(kda::kModeFixup, bf, dk, dv, nbf, f, s),
                    "prefill split (fix-up)");
}

// Segments whose (segment, head) units would leave compute units idle (or run
// with half-width value blocks that repeat the producer work) are split into
// f sub-segments of at least kMinSubSplit tokens on average; their packages
// are merged in the workspace (kda_segment_package).
constexpr int64_t kMinSubSplit = 512;

struct PackageSplit {
    int f = 1;
    size_t off_sb = 0, off_ord = 0, off_M = 0, off_D = 0, off_X = 0, off_Xlen = 0, off_Pi = 0,
           off_route = 0, bytes = 0;
    bool fixop = false;   // the later sub-segments keep their fix-up operators
};

bool plan_package_split(const kda_config *cfg, int64_t T, int32_t nseg, PackageSplit *p,
                        bool fixop = true) {
    if (nseg <= 0 || T <= 0) return false;
    const int64_t units = (int64_t)nseg * cfg->num_heads;
    const int cus = device_cus();
    if (units >= cus) return false;
    int64_t f = (cus + units - 1) / units;
    f = std::min<int64_t>(f, 8);
    f = std::min<int64_t>(f, T / nseg / kMinSubSplit);
    if (f < 2) return false;
    p->f = (int)f;
    const size_t nsub = (size_t)f * nseg, H = (size_t)cfg->num_heads;
    size_t at = 0;
    auto take = [&](size_t b) { const size_t o = at; at += round256(b); return o; };
    p->off_sb = take(sizeof(int64_t) * (nsub + 1));
    p->off_ord = take(sizeof(int32_t) * (size_t)(f - 1) * nseg);
    p->off_M = take(sizeof(float) * nsub * H * cfg->dk * cfg->dk);
    p->off_D = take(sizeof(float) * nsub * H * cfg->dk * cfg->dv);
    // the fix-up operators of sub-segments 1..f-1 (the chunked engine's shapes only)
    const bool bf = cfg->io_dtype == KDA_DTYPE_BF16;
    p->fixop = fixop && !kda::recurrent_supported(bf, cfg->dk, cfg->dv);
    if (p->fixop) {
        const size_t later = (size_t)(f - 1) * nseg, io = bf ? 2 : 4;
        p->off_X = take(later * kSplitFixopChunks * kda::kChunk * H * cfg->dk * io);
        p->off_Xlen = take(later * H * (cfg->dk / 64) * sizeof(int32_t));
        p->off_Pi = take(later * H * cfg->dk * cfg->dk * sizeof(float));
        p->off_route = take(nsub * H * sizeof(int32_t));
    }
    p->bytes = at;
    return true;
}

int package_split(const PackageSplit &p, const kda_config *cfg, const void *q, const void *k,
                  const void *v, const float *g, const float *beta, int64_t T,
                  const int64_t *seg_start, int32_t nseg, void *o_local, float *M, float *D,
                  int32_t interval, float *sub_M, float *sub_D, const kda_fixop *fxo, void *ws,
                  hipStream_t s) {
    unsigned char *w = (unsigned char *)ws;
    int64_t *sb = (int64_t *)(w + p.off_sb);
    int32_t *ord = (int32_t *)(w + p.off_ord);
    float *Ms = (float *)(w + p.off_M), *Ds = (float *)(w + p.off_D);
    const bool bf = cfg->io_dtype == KDA_DTYPE_BF16;
    const int H = cfg->num_heads, dk = cfg->dk, dv = cfg->dv, f = p.f;
    const int nsub = f * nseg;
    hipError_t e = kda::launch_split_bounds(seg_start, nseg, f, sb, ord, s);
    if (e != hipSuccess) return launched(e, "package split (bounds)");
    // packages of every sub-segment, M included (the merge needs it)
    const int nb = kda::engine_pick_nb(bf, dk, dv, (int64_t)nsub * H, kda::kModePackage);
    kda::EngineArgs a{};
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.o = o_local;
    a.bounds = sb; a.order = nullptr; a.n_units = nsub; a.H = H;
    a.S_init = nullptr; a.S_out = Ds; a.M_out = Ms;
    a.interval = interval; a.ckpt_off = nullptr; a.ckpt_S = sub_D; a.ckpt_M = sub_M;
    a.scale = cfg->scale; a.l2norm = cfg->qk_l2norm;
    a.ncb = dv / nb;
    a.ncb_m = dk / std::min(nb, dk);
    a.X_per = f;
    a.S_last = D; a.M_last = M;   // the last sub-segments' packages: where the merge ends
    if (fxo) {   // the operator of each segment from its first sub-segment's M blocks
        a.X = fxo->X; a.X_len = fxo->len; a.X_chunks = fxo->chunks;
        a.X_Pi = fxo->interval > 0 ? fxo->Pi : nullptr; a.X_interval = fxo->interval;
    }
    const bool rung_pi = interval > 0 && sub_D;
    const size_t x_slot = (size_t)kSplitFixopChunks * kda::kChunk * H * dk * (bf ? 2 : 4);
    if (p.fixop) {   // and the operators of the later sub-segments, for the merge below
        a.Xs = w + p.off_X; a.Xs_len = (int32_t *)(w + p.off_Xlen);
        a.Xs_chunks = kSplitFixopChunks;
        if (rung_pi) {
            a.Xs_Pi = (float *)(w + p.off_Pi); a.Xs_interval = interval;
        }
    }
    if ((e = kda::launch_engine(kda::kModePackageVM, bf, dk, dv, nb, a, s)) != hipSuccess)
        return launched(e, "package split (packages)");
    const int nbf = kda::engine_pick_nb(bf, dk, dv, (int64_t)nseg * H, kda::kModeFixup);
    const size_t slot = (size_t)H * dk * dv;
    for (int kk = 1; kk < f; ++kk) {
        // sub-segment kk of every segment fixed up from the accumulated state
        // of sub-segments 0..kk-1, kept in the slot before it (S_init[u] = Ds[u-1])
        kda::EngineArgs fx{};
        fx.q = q; fx.k = k; fx.v = nullptr; fx.g = g; fx.beta = beta; fx.o = o_local;
        fx.bounds = sb; fx.order = ord + (size_t)(kk - 1) * nseg; fx.n_units = nseg; fx.H = H;
        fx.S_init = (const float *)((uintptr_t)Ds - slot * sizeof(float));
        fx.scale = cfg->scale; fx.l2norm = cfg->qk_l2norm;
        if (rung_pi) {   // rungs inside it: in place
            fx.interval = interval; fx.ckpt_S = sub_D; fx.ckpt_in = sub_D;
        }
        fx.ncb = dv / nbf;
        if (p.fixop) {   // the sub-segments their operators cover, then the recurrence for the rest
            const size_t at = (size_t)(kk - 1) * nseg;
            kda::EngineArgs x = fx;
            x.X = w + p.off_X + at * x_slot;
            x.X_len = (int32_t *)(w + p.off_Xlen) + at * H * (dk / 64);
            x.X_chunks = kSplitFixopChunks;
            if (rung_pi) {
                x.X_Pi = (float *)(w + p.off_Pi) + at * H * dk * dk; x.X_interval = interval;
            }
            x.X_route = (int32_t *)(w + p.off_route);
            if ((e = kda::launch_engine(kda::kModeFixOp, bf, dk, dv, nbf, x, s)) != hipSuccess)
                return launched(e, "package split (fix-up operator)");
            fx.X_route = x.X_route;
        }
        if ((e = kda::launch_engine(kda::kModeFixup, bf, dk, dv, nbf, fx, s)) != hipSuccess)
            return launched(e, "package split (fix-up)");
        if (interval > 0 && sub_M) {
            e = kda::launch_split_rung_m(dk, H, nseg, f, kk, sb, interval, T / interval, Ms, sub_M, s);
            if (e != hipSuccess) return launched(e, "package split (rungs)");
        }
        if ((e = kda::launch_split_compose(dk, dv, H, nseg, f, kk, Ms, Ds, M, D, s)) != hipSuccess)
            return launched(e, "package split (compose)");
    }
    return ok();
}

// Scratch of kda_prefill_noalloc: one fixed array per device, held for the
// life of the process, in place of the caller's workspace.  In host code the
// array's name only stands in for the symbol; the device address of each
// device's copy comes from hipGetSymbolAddress, called once per device with
// that device current, and only that address is handed to kernels.
static __device__ __align__(256) unsigned char scratch[KDA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

int scratch_address(void **out) {
    static std::mutex mu;
    static void *addr[kMaxDevices] = {};
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(KDA_ERR_DEVICE, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(KDA_ERR_UNSUPPORTED, "device index %d beyond the %d the library tracks", dev,
                    kMaxDevices);
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(KDA_ERR_DEVICE, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                        hipGetErrorString(e));
        addr[dev] = p;
    }
    *out = addr[dev];
    return KDA_OK;
}

// Chunked prefill with initial / final states either dense (S0, S_final) or
// in a slot pool; pos0 (nullable) shifts the checkpoint grid.
int prefill_impl(const char *what, const kda_config *cfg, const void *q, const void *k,
                 const void *v, const float *g, const float *beta, const int64_t *cu_seqlens,
                 int32_t N, int64_t T, const float *S0, float *S_final,
                 const kda_state_pool *pool, const int64_t *pos0, void *o, const kda_ckpt *ckpt,
                 void *ws, size_t ws_bytes, void *stream, bool noalloc = false) {
    KDA_TRY(check_config(cfg));
    if (T < 0) return fail(KDA_ERR_ARG, "T must be >= 0 (got %lld)", (long long)T);
    if (N < 0) return fail(KDA_ERR_ARG, "N must be >= 0 (got %d)", N);
    if (T > 0 && N == 0) return fail(KDA_ERR_ARG, "T > 0 needs at least one sequence");
    if (pool) {
        if (pool->n_slots <= 0)
            return fail(KDA_ERR_ARG, "pool->n_slots must be positive (got %lld)",
                        (long long)pool->n_slots);
        KDA_TRY(check_tensor(pool->states, "pool->states", true, 16));
        KDA_TRY(check_tensor(pool->read_idx, "pool->read_idx", N > 0, 4));
        KDA_TRY(check_tensor(pool->write_idx, "pool->write_idx", N > 0, 4));
    }
    KDA_TRY(check_tensor(pos0, "pos0", false, 8));
    if (N == 0) return ok();
    const bool need_rows = T > 0;
    KDA_TRY(check_tensor(q, "q", need_rows));
    KDA_TRY(check_tensor(k, "k", need_rows));
    KDA_TRY(check_tensor(v, "v", need_rows));
    KDA_TRY(check_tensor(g, "g", need_rows));
    KDA_TRY(check_tensor(beta, "beta", need_rows, 4));
    KDA_TRY(check_tensor(o, "o", need_rows));
    KDA_TRY(check_tensor(cu_seqlens, "cu_seqlens", true, 8));
    KDA_TRY(check_tensor(S0, "S0", false, 16));
    KDA_TRY(check_tensor(S_final, "S_final", false, 16));
    if (ckpt) {
        KDA_TRY(check_ckpt_interval(ckpt->interval));
        KDA_TRY(check_tensor(ckpt->states, "ckpt->states", true, 16));
        KDA_TRY(check_tensor(ckpt->offsets, "ckpt->offsets", N > 1, 8));
    }
    const size_t need = prefill_ws_bytes(N);
    if (noalloc) {
        // the library's fixed scratch stands in for the workspace
        if (need > (size_t)KDA_NOALLOC_SCRATCH_BYTES)
            return fail(KDA_ERR_WORKSPACE,
                        "N = %d sequences need %zu bytes of scratch, more than the fixed %zu", N,
                        need, (size_t)KDA_NOALLOC_SCRATCH_BYTES);
        KDA_TRY(scratch_address(&ws));
        ws_bytes = KDA_NOALLOC_SCRATCH_BYTES;
    }
    if (!ws || ws_bytes < need)
        return fail(KDA_ERR_WORKSPACE, "workspace of %zu bytes required (got %zu)", need, ws_bytes);
    KDA_TRY(check_tensor(ws, "ws", true, 16));

    hipStream_t s = (hipStream_t)stream;
    SplitPlan sp;
    // the segmented path, with the fix-up operator when the workspace holds it
    if (!pool && !pos0 && plan_split(cfg, T, N, ckpt, &sp) &&
        (ws_bytes >= sp.bytes || (plan_split(cfg, T, N, ckpt, &sp, false) && ws_bytes >= sp.bytes)))
        return prefill_split(sp, cfg, q, k, v, g, beta, T, S0, S_final, o, ckpt, ws, s);
    const bool bf = cfg->io_dtype == KDA_DTYPE_BF16;
    const int nb = kda::engine_pick_nb(bf, cfg->dk, cfg->dv, (int64_t)N * cfg->num_heads,
                                       kda::kModePrefill);
    int32_t *order = nullptr;
    if (N > 1 && N <= 8192) {
        order = (int32_t *)ws;
        hipError_t e = kda::launch_plan(cu_seqlens, N, order, s);
        if (e != hipSuccess) return launched(e, "plan");
    }
    kda::EngineArgs a{};
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.o = o;
    a.bounds = cu_seqlens; a.order = order; a.n_units = N; a.H = cfg->num_heads;
    a.ncb = cfg->dv / nb;
    a.S_init = pool ? pool->states : S0;
    a.S_out = pool ? pool->states : S_final;
    a.M_out = nullptr;
    a.interval = ckpt ? ckpt->interval : 0;
    a.ckpt_off = ckpt ? ckpt->offsets : nullptr;
    a.ckpt_S = ckpt ? ckpt->states : nullptr;
    a.ckpt_M = nullptr;
    a.scale = cfg->scale; a.l2norm = cfg->qk_l2norm;
    a.s_in_idx = pool ? pool->read_idx : nullptr;
    a.s_out_idx = pool ? pool->write_idx : nullptr;
    a.n_slots = pool ? pool->n_slots : 0;
    a.pos0 = pos0;
    return launched(kda::launch_engine(kda::kModePrefill, bf, cfg->dk, cfg->dv, nb, a, s), what);
}

}  // namespace

extern "C" {

const char *kda_status_string(int status) {
    switch (status) {
        case KDA_OK: return "KDA_OK";
        case KDA_ERR_ARG: return "KDA_ERR_ARG: invalid argument";
        case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED: shape or dtype not built";
        case KDA_ERR_ALIGN: return "KDA_ERR_ALIGN: misaligned device pointer";
        case KDA_ERR_WORKSPACE: return "KDA_ERR_WORKSPACE: workspace missing or too small";
        case KDA_ERR_DEVICE: return "KDA_ERR_DEVICE: kernel launch failed";
    }
    return "unknown KDA status";
}

const char *kda_last_error(void) { return g_last_error.c_str(); }

int kda_validate_inputs(const kda_config *cfg, int64_t T, const int64_t *bounds, int32_t n,
                        int32_t chunk_aligned, const float *g, const float *beta,
                        int32_t *report, void *stream) {
    KDA_TRY(check_config(cfg));
    if (T < 0) return fail(KDA_ERR_ARG, "T must be >= 0 (got %lld)", (long long)T);
    if (bounds && n < 1) return fail(KDA_ERR_ARG, "n must be >= 1 with bounds (got %d)", n);
    if (chunk_aligned != 0 && chunk_aligned != 1)
        return fail(KDA_ERR_ARG, "chunk_aligned must be 0 or 1 (got %d)", chunk_aligned);
    KDA_TRY(check_tensor(report, "report", true, 4));
    KDA_TRY(check_tensor(bounds, "bounds", false, 8));
    KDA_TRY(check_tensor(g, "g", false));
    KDA_TRY(check_tensor(beta, "beta", false, 4));
    return launched(kda::launch_validate(T, cfg->num_heads, cfg->dk, bounds, bounds ? n : 0,
                                         chunk_aligned, g, beta, report, KDA_CHECK_FIELDS,
                                         (hipStream_t)stream),
                    "input validation");
}

const char *kda_version(void) { return "0.1.0"; }

size_t kda_prefill_workspace(const kda_config *cfg, int64_t T, int32_t N) {
    size_t need = prefill_ws_bytes(N);
    SplitPlan sp;
    // room for the segmented path of a call without checkpoints
    if (cfg && check_config(cfg) == KDA_OK && plan_split(cfg, T, N, nullptr, &sp))
        need = std::max(need, sp.bytes);
    return need;
}

int kda_prefill(const kda_config *cfg, const void *q, const void *k, const void *v,
                const float *g, const float *beta, const int64_t *cu_seqlens, int32_t N,
                int64_t T, const float *S0, float *S_final, void *o, const kda_ckpt *ckpt,
                void *ws, size_t ws_bytes, void *stream) {
    return prefill_impl("prefill", cfg, q, k, v, g, beta, cu_seqlens, N, T, S0, S_final, nullptr,
                        nullptr, o, ckpt, ws, ws_bytes, stream);
}

int kda_prefill_noalloc(const kda_config *cfg, const void *q, const void *k, const void *v,
                        const float *g, const float *beta, const int64_t *cu_seqlens, int32_t N,
                        int64_t T, const float *S0, float *S_final, void *o, const kda_ckpt *ckpt,
                        void *stream) {
    // arguments are checked first; the scratch then stands in for a caller's
    // workspace of KDA_NOALLOC_SCRATCH_BYTES (the one-pass schedule needs N
    // int32 entries, the segmented path of one sequence runs when it fits)
    return prefill_impl("prefill (no allocation)", cfg, q, k, v, g, beta, cu_seqlens, N, T, S0,
                        S_final, nullptr, nullptr, o, ckpt, nullptr, 0, stream, true);
}

int kda_prefill_resume(const kda_config *cfg, const void *q, const void *k, const void *v,
                       const float *g, const float *beta, const int64_t *cu_seqlens, int32_t N,
                       int64_t T, const int64_t *pos0, const kda_state_pool *pool, void *o,
                       const kda_ckpt *ckpt, void *ws, size_t ws_bytes, void *stream) {
    if (!pool) return fail(KDA_ERR_ARG, "pool is NULL");
    return prefill_impl("prefill resume", cfg, q, k, v, g, beta, cu_seqlens, N, T, nullptr,
                        nullptr, pool, pos0, o, ckpt, ws, ws_bytes, stream);
}

size_t kda_segment_package_workspace(const kda_config *cfg, int64_t T, int32_t nseg) {
    PackageSplit p;
    if (!cfg || check_config(cfg) != KDA_OK || !plan_package_split(cfg, T, nseg, &p)) return 0;
    return p.bytes;
}

// Arguments of a fix-up operator (kda_fixop) for the chunked engine's shapes.
int check_fixop(const kda_config *cfg, const kda_fixop *fx) {
    if (fx->chunks <= 0) return fail(KDA_ERR_ARG, "fx->chunks must be positive (got %d)", fx->chunks);
    KDA_TRY(check_tensor(fx->X, "fx->X", true));
    KDA_TRY(check_tensor(fx->len, "fx->len", true, 4));
    KDA_TRY(check_tensor(fx->route, "fx->route", true, 4));
    KDA_TRY(check_tensor(fx->Pi, "fx->Pi", false));
    if (fx->interval < 0) return fail(KDA_ERR_ARG, "fx->interval must be >= 0 (got %d)", fx->interval);
    if (fx->interval > 0) KDA_TRY(check_ckpt_interval(fx->interval));
    if (kda::recurrent_supported(cfg->io_dtype == KDA_DTYPE_BF16, cfg->dk, cfg->dv))
        return fail(KDA_ERR_UNSUPPORTED, "a fix-up operator needs the chunked engine "
                                         "(not fp32 I/O with dk = 128)");
    return KDA_OK;
}

int package_impl(const kda_config *cfg, const void *q, const void *k, const void *v,
                 const float *g, const float *beta, int64_t T, const int64_t *seg_start,
                 int32_t nseg, void *o_local, float *M, float *D, const kda_ckpt *ckpt,
                 float *sub_M, float *sub_D, const kda_fixop *fx, void *ws, size_t ws_bytes,
                 void *stream) {
    KDA_TRY(check_config(cfg));
    if (T <= 0) return fail(KDA_ERR_ARG, "T must be positive (got %lld)", (long long)T);
    if (nseg <= 0) return fail(KDA_ERR_ARG, "nseg must be positive (got %d)", nseg);
    KDA_TRY(check_tensor(q, "q", true));
    KDA_TRY(check_tensor(k, "k", true));
    KDA_TRY(check_tensor(v, "v", true));
    KDA_TRY(check_tensor(g, "g", true));
    KDA_TRY(check_tensor(beta, "beta", true, 4));
    KDA_TRY(check_tensor(o_local, "o_local", true));
    KDA_TRY(check_tensor(seg_start, "seg_start", true, 8));
    KDA_TRY(check_tensor(M, "M", false));
    KDA_TRY(check_tensor(D, "D", true));
    const bool subs = ckpt && (sub_M || sub_D);
    if (subs) {
        KDA_TRY(check_ckpt_interval(ckpt->interval));
        KDA_TRY(check_tensor(sub_M, "sub_M", false));
        KDA_TRY(check_tensor(sub_D, "sub_D", true));
        if (sub_M && !M) return fail(KDA_ERR_ARG, "sub_M needs M (M is NULL)");
    }
    if (fx) {
        KDA_TRY(check_fixop(cfg, fx));
        if (!M) return fail(KDA_ERR_ARG, "a fix-up operator needs M (M is NULL)");
    }
    hipStream_t s = (hipStream_t)stream;
    PackageSplit sp;
    // the split with the sub-segments' fix-up operators, else without them
    // when the workspace holds only that
    if (ws && ((plan_package_split(cfg, T, nseg, &sp) && ws_bytes >= sp.bytes) ||
               (plan_package_split(cfg, T, nseg, &sp, false) && ws_bytes >= sp.bytes))) {
        KDA_TRY(check_tensor(ws, "ws", true));
        return package_split(sp, cfg, q, k, v, g, beta, T, seg_start, nseg, o_local, M, D,
                             subs ? ckpt->interval : 0, subs ? sub_M : nullptr,
                             subs ? sub_D : nullptr, fx, ws, s);
    }
    const bool bf = cfg->io_dtype == KDA_DTYPE_BF16;
    const int nb = kda::engine_pick_nb(bf, cfg->dk, cfg->dv, (int64_t)nseg * cfg->num_heads,
                                       kda::kModePackage);
    kda::EngineArgs a{};
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.o = o_local;
    a.bounds = seg_start; a.order = nullptr; a.n_units = nseg; a.H = cfg->num_heads;
    a.S_init = nullptr; a.S_out = D; a.M_out = M;
    a.interval = subs ? ckpt->interval : 0;
    a.ckpt_off = nullptr; a.ckpt_S = subs ? sub_D : nullptr; a.ckpt_M = subs ? sub_M : nullptr;
    a.scale = cfg->scale; a.l2norm = cfg->qk_l2norm;
    if (fx) {
        a.X = fx->X; a.X_len = fx->len; a.X_chunks = fx->chunks;
        a.X_Pi = fx->interval > 0 ? fx->Pi : nullptr; a.X_interval = fx->interval;
    }
    // Value blocks, and with M the M blocks after them in the same grid (they
    // stop as soon as M is exactly zero and fill the value blocks' tail).
    a.ncb = cfg->dv / nb;
    a.ncb_m = cfg->dk / std::min(nb, cfg->dk);   // M has dk columns
    return launched(kda::launch_engine(M ? kda::kModePackageVM : kda::kModePackage, bf, cfg->dk,
                                       cfg->dv, nb, a, s), "package");
}

int kda_segment_package(const kda_config *cfg, const void *q, const void *k, const void *v,
                        const float *g, const float *beta, int64_t T, const int64_t *seg_start,
                        int32_t nseg, void *o_local, float *M, float *D, const kda_ckpt *ckpt,
                        float *sub_M, float *sub_D, void *ws, size_t ws_bytes, void *stream) {
    return package_impl(cfg, q, k, v, g, beta, T, seg_start, nseg, o_local, M, D, ckpt, sub_M,
                        sub_D, nullptr, ws, ws_bytes, stream);
}

int kda_segment_package_fx(const kda_config *cfg, const void *q, const void *k, const void *v,
                           const float *g, const float *beta, int64_t T,
                           const int64_t *seg_start, int32_t nseg, void *o_local, float *M,
                           float *D, const kda_ckpt *ckpt, float *sub_M, float *sub_D,
                           const kda_fixop *fx, void *ws, size_t ws_bytes, void *stream) {
    if (!fx) return fail(KDA_ERR_ARG, "fx is NULL");
    return package_impl(cfg, q, k, v, g, beta, T, seg_start, nseg, o_local, M, D, ckpt, sub_M,
                        sub_D, fx, ws, ws_bytes, stream);
}

size_t kda_segment_scan_workspace(const kda_config *cfg, int32_t nseg, int32_t algo) {
    if (!cfg || nseg <= 0 || cfg->num_heads <= 0) return 0;
    if (algo == KDA_SCAN_SEQUENTIAL) return round256(kda::sequential_workspace(cfg->num_heads, nseg));
    if (algo != KDA_SCAN_BLELLOCH) return 0;
    return round256(kda::blelloch_workspace(cfg->dk, cfg->dv, cfg->num_heads, nseg));
}

int kda_segment_scan(const kda_config *cfg, int32_t nseg, const float *M, const float *D,
                     const float *S0, float *S_in, float *S_final, int32_t algo, void *ws,
                     size_t ws_bytes, void *stream) {
    KDA_TRY(check_config(cfg));
    if (nseg <= 0) return fail(KDA_ERR_ARG, "nseg must be positive (got %d)", nseg);
    if (algo != KDA_SCAN_SEQUENTIAL && algo != KDA_SCAN_BLELLOCH)
        return fail(KDA_ERR_ARG, "algo must be KDA_SCAN_SEQUENTIAL or KDA_SCAN_BLELLOCH (got %d)", algo);
    KDA_TRY(check_tensor(M, "M", true));
    KDA_TRY(check_tensor(D, "D", true));
    KDA_TRY(check_tensor(S0, "S0", false));
    KDA_TRY(check_tensor(S_in, "S_in", true));
    KDA_TRY(check_tensor(S_final, "S_final", true));
    hipStream_t s = (hipStream_t)stream;
    if (algo == KDA_SCAN_SEQUENTIAL) {   // the workspace is optional: M tested once per package
        const bool flags = ws && ws_bytes >= kda::sequential_workspace(cfg->num_heads, nseg);
        if (flags) KDA_TRY(check_tensor(ws, "ws", true, 4));
        return launched(kda::launch_scan_sequential(cfg->dk, cfg->dv, cfg->num_heads, nseg, M, D,
                                                    S0, S_in, S_final, flags ? (int *)ws : nullptr,
                                                    s),
                        "sequential scan");
    }
    if (nseg > kda::blelloch_max_segments())
        return fail(KDA_ERR_UNSUPPORTED, "the Blelloch scan takes at most %d segments (got %d)",
                    kda::blelloch_max_segments(), nseg);
    const size_t need = kda_segment_scan_workspace(cfg, nseg, algo);
    if (!ws || ws_bytes < need)
        return fail(KDA_ERR_WORKSPACE, "workspace of %zu bytes required (got %zu)", need, ws_bytes);
    KDA_TRY(check_tensor(ws, "ws", true));
    return launched(kda::launch_scan_blelloch(cfg->dk, cfg->dv, cfg->num_heads, nseg, M, D, S0,
                                              S_in, S_final, ws, s), "Blelloch scan");
}

int kda_output_fixup(const kda_config *cfg, const void *q, const void *k, const float *g,
                     const float *beta, int64_t T, const int64_t *seg_start, int32_t nseg,
                     const float *S_in, void *o, void *ws, size_t ws_bytes, void *stream) {
    return kda_output_fixup_ckpt(cfg, q, k, g, beta, T, seg_start, nseg, S_in, o, nullptr,
                                 nullptr, ws, ws_bytes, stream);
}

int fixup_impl(const kda_config *cfg, const void *q, const void *k, const float *g,
               const float *beta, int64_t T, const int64_t *seg_start, int32_t nseg,
               const float *S_in, void *o, const kda_ckpt *ckpt, const float *sub_D,
               const kda_fixop *fx, void *stream) {
    KDA_TRY(check_config(cfg));
    if (fx) KDA_TRY(check_fixop(cfg, fx));
    if (ckpt) {
        KDA_TRY(check_ckpt_interval(ckpt->interval));
        KDA_TRY(check_tensor(ckpt->states, "ckpt->states", true));
        KDA_TRY(check_tensor(sub_D, "sub_D", true));
    }
    if (T <= 0) return fail(KDA_ERR_ARG, "T must be positive (got %lld)", (long long)T);
    if (nseg <= 0) return fail(KDA_ERR_ARG, "nseg must be positive (got %d)", nseg);
    KDA_TRY(check_tensor(q, "q", true));
    KDA_TRY(check_tensor(k, "k", true));
    KDA_TRY(check_tensor(g, "g", true));
    KDA_TRY(check_tensor(beta, "beta", true, 4));
    KDA_TRY(check_tensor(seg_start, "seg_start", true, 8));
    KDA_TRY(check_tensor(S_in, "S_in", true));
    KDA_TRY(check_tensor(o, "o", true));
    hipStream_t s = (hipStream_t)stream;
    const bool bf = cfg->io_dtype == KDA_DTYPE_BF16;
    const int nb = kda::engine_pick_nb(bf, cfg->dk, cfg->dv, (int64_t)nseg * cfg->num_heads,
                                       kda::kModeFixup);
    kda::EngineArgs a{};
    a.q = q; a.k = k; a.v = nullptr; a.g = g; a.beta = beta; a.o = o;
    a.bounds = seg_start; a.order = nullptr; a.n_units = nseg; a.H = cfg->num_heads;
    a.ncb = cfg->dv / nb;
    a.S_init = S_in; a.S_out = nullptr; a.M_out = nullptr;
    a.interval = ckpt ? ckpt->interval : 0; a.ckpt_off = nullptr;
    a.ckpt_S = ckpt ? ckpt->states : nullptr; a.ckpt_in = ckpt ? sub_D : nullptr;
    a.ckpt_M = nullptr;
    a.scale = cfg->scale; a.l2norm = cfg->qk_l2norm;
    if (fx) {   // the units the operator covers first; the launch below skips them
        kda::EngineArgs x = a;
        x.X = fx->X; x.X_len = fx->len; x.X_chunks = fx->chunks; x.X_route = fx->route;
        x.X_Pi = fx->interval > 0 ? fx->Pi : nullptr; x.X_interval = fx->interval;
        hipError_t e = kda::launch_engine(kda::kModeFixOp, bf, cfg->dk, cfg->dv, nb, x, s);
        if (e != hipSuccess) return launched(e, "fixup (operator)");
        a.X_route = fx->route;
    }
    return launched(kda::launch_engine(kda::kModeFixup, bf, cfg->dk, cfg->dv, nb, a, s), "fixup");
}

int kda_output_fixup_ckpt(const kda_config *cfg, const void *q, const void *k, const float *g,
                          const float *beta, int64_t T, const int64_t *seg_start, int32_t nseg,
                          const float *S_in, void *o, const kda_ckpt *ckpt, const float *sub_D,
                          void *ws, size_t ws_bytes, void *stream) {
    (void)ws;
    (void)ws_bytes;
    return fixup_impl(cfg, q, k, g, beta, T, seg_start, nseg, S_in, o, ckpt, sub_D, nullptr,
                      stream);
}

int kda_output_fixup_fx(const kda_config *cfg, const void *q, const void *k, const float *g,
                        const float *beta, int64_t T, const int64_t *seg_start, int32_t nseg,
                        const float *S_in, void *o, const kda_ckpt *ckpt, const float *sub_D,
                        const kda_fixop *fx, void *stream) {
    return fixup_impl(cfg, q, k, g, beta, T, seg_start, nseg, S_in, o, ckpt, sub_D, fx, stream);
}

int kda_checkpoint_write(const kda_config *cfg, const kda_ckpt *ckpt, int64_t T,
                         const int64_t *seg_start, int32_t nseg, const float *S_in,
                         const float *sub_M, const float *sub_D, void *stream) {
    KDA_TRY(check_config(cfg));
    if (!ckpt) return fail(KDA_ERR_ARG, "ckpt is NULL");
    KDA_TRY(check_ckpt_interval(ckpt->interval));
    if (T <= 0) return fail(KDA_ERR_ARG, "T must be positive (got %lld)", (long long)T);
    if (nseg <= 0) return fail(KDA_ERR_ARG, "nseg must be positive (got %d)", nseg);
    KDA_TRY(check_tensor(ckpt->states, "ckpt->states", true));
    KDA_TRY(check_tensor(seg_start, "seg_start", true, 8));
    KDA_TRY(check_tensor(S_in, "S_in", true));
    KDA_TRY(check_tensor(sub_M, "sub_M", true));
    KDA_TRY(check_tensor(sub_D, "sub_D", true));
    return launched(kda::launch_ckpt_write(cfg->dk, cfg->dv, cfg->num_heads, T, seg_start, nseg,
                                           ckpt->interval, S_in, sub_M, sub_D, ckpt->states,
                                           (hipStream_t)stream), "checkpoint write");
}

int kda_decode(const kda_config *cfg, int32_t N, const void *q, const void *k, const void *v,
               const float *g, const float *beta, int32_t gate_logits,
               const kda_state_pool *pool, void *o, void *stream) {
    KDA_TRY(check_config(cfg, true));
    if (N < 0) return fail(KDA_ERR_ARG, "N must be non-negative (got %d)", N);
    if (gate_logits != 0 && gate_logits != 1)
        return fail(KDA_ERR_ARG, "gate_logits must be 0 or 1 (got %d)", gate_logits);
    if (!pool) return fail(KDA_ERR_ARG, "pool is NULL");
    if (pool->n_slots <= 0)
        return fail(KDA_ERR_ARG, "pool->n_slots must be positive (got %lld)", (long long)pool->n_slots);
    if (N == 0) return ok();
    if ((int64_t)N * cfg->num_heads * (cfg->dv / 64) > INT32_MAX)
        return fail(KDA_ERR_UNSUPPORTED, "N * num_heads is too large for one launch");
    KDA_TRY(check_tensor(q, "q", true));
    KDA_TRY(check_tensor(k, "k", true));
    KDA_TRY(check_tensor(v, "v", true));
    KDA_TRY(check_tensor(g, "g", true));
    KDA_TRY(check_tensor(beta, "beta", true, 4));
    KDA_TRY(check_tensor(o, "o", true));
    KDA_TRY(check_tensor(pool->states, "pool->states", true, 16));
    KDA_TRY(check_tensor(pool->read_idx, "pool->read_idx", true, 4));
    KDA_TRY(check_tensor(pool->write_idx, "pool->write_idx", true, 4));
    kda::DecodeArgs a{};
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.o = o;
    a.pool = pool->states; a.n_slots = pool->n_slots;
    a.read_idx = pool->read_idx; a.write_idx = pool->write_idx;
    a.N = N; a.H = cfg->num_heads; a.scale = cfg->scale; a.l2norm = cfg->qk_l2norm;
    a.gate_logits = gate_logits;
    return launched(kda::launch_decode(cfg->io_dtype == KDA_DTYPE_BF16, cfg->dk, cfg->dv, a,
                                       (hipStream_t)stream), "decode");
}

}  // extern "C"

namespace {

int check_conv_common(int32_t io_dtype, int32_t channels, int32_t width, const void *x, int64_t T) {
    if (io_dtype != KDA_DTYPE_F32 && io_dtype != KDA_DTYPE_BF16)
        return fail(KDA_ERR_ARG, "io_dtype must be KDA_DTYPE_F32 or KDA_DTYPE_BF16 (got %d)", io_dtype);
    if (channels <= 0 || channels % 8 != 0)
        return fail(KDA_ERR_UNSUPPORTED, "channels must be a positive multiple of 8 (got %d)", channels);
    if (width < 2 || width > 8)
        return fail(KDA_ERR_UNSUPPORTED, "width must be in [2, 8] (got %d)", width);
    if (T < 0) return fail(KDA_ERR_ARG, "T must be >= 0 (got %lld)", (long long)T);
    KDA_TRY(check_tensor(x, "x", T > 0));
    return KDA_OK;
}

int check_conv_state(const kda_conv_state *st) {
    if (!st) return KDA_OK;
    if (st->n_slots <= 0)
        return fail(KDA_ERR_ARG, "state->n_slots must be positive (got %lld)", (long long)st->n_slots);
    KDA_TRY(check_tensor(st->states, "state->states", true));
    KDA_TRY(check_tensor(st->read_idx, "state->read_idx", false, 4));
    KDA_TRY(check_tensor(st->write_idx, "state->write_idx", false, 4));
    return KDA_OK;
}

}  // namespace

extern "C" {

int kda_short_conv(int32_t io_dtype, int32_t channels, int32_t width, int32_t activation,
                   const void *x, int64_t T, const int64_t *cu_seqlens, int32_t N,
                   const float *weight, const float *bias, const kda_conv_state *state, void *y,
                   void *stream) {
    KDA_TRY(check_conv_common(io_dtype, channels, width, x, T));
    if (activation != KDA_ACT_NONE && activation != KDA_ACT_SILU)
        return fail(KDA_ERR_ARG, "activation must be KDA_ACT_NONE or KDA_ACT_SILU (got %d)", activation);
    if (N < 0) return fail(KDA_ERR_ARG, "N must be >= 0 (got %d)", N);
    if (T > 0 && N == 0) return fail(KDA_ERR_ARG, "T > 0 needs at least one sequence");
    if ((T + 63) / 64 > INT32_MAX) return fail(KDA_ERR_UNSUPPORTED, "T is too large for one launch");
    KDA_TRY(check_conv_state(state));
    if (N == 0) return ok();
    KDA_TRY(check_tensor(cu_seqlens, "cu_seqlens", true, 8));
    KDA_TRY(check_tensor(weight, "weight", true, 4));
    KDA_TRY(check_tensor(bias, "bias", false, 4));
    KDA_TRY(check_tensor(y, "y", T > 0));
    if (T > 0 && x == y) return fail(KDA_ERR_ARG, "y must not alias x");
    kda::ConvArgs a{};
    a.x = x; a.y = y; a.weight = weight; a.bias = bias; a.cu = cu_seqlens;
    a.N = N; a.C = channels; a.T = T; a.act = activation;
    a.win = state ? state->states : nullptr;
    a.n_slots = state ? state->n_slots : 0;
    a.read_idx = state ? state->read_idx : nullptr;
    a.write_idx = state ? state->write_idx : nullptr;
    return launched(kda::launch_conv(io_dtype == KDA_DTYPE_BF16, width, a, (hipStream_t)stream),
                    "short conv");
}

int kda_conv_halo(int32_t io_dtype, int32_t channels, int32_t width, const void *x, int64_t T,
                  const int64_t *bounds, int32_t nseg, const kda_conv_state *dst, void *stream) {
    KDA_TRY(check_conv_common(io_dtype, channels, width, x, T));
    if (nseg < 0) return fail(KDA_ERR_ARG, "nseg must be >= 0 (got %d)", nseg);
    if (!dst) return fail(KDA_ERR_ARG, "dst is NULL");
    KDA_TRY(check_conv_state(dst));
    if (nseg == 0) return ok();
    KDA_TRY(check_tensor(dst->write_idx, "dst->write_idx", true, 4));
    KDA_TRY(check_tensor(bounds, "bounds", true, 8));
    kda::ConvArgs a{};
    a.x = x; a.cu = bounds; a.N = nseg; a.C = channels; a.T = T;
    a.win = dst->states; a.n_slots = dst->n_slots; a.write_idx = dst->write_idx;
    return launched(kda::launch_conv_halo(io_dtype == KDA_DTYPE_BF16, width, a, (hipStream_t)stream),
                    "conv halo");
}

}  // extern "C"
