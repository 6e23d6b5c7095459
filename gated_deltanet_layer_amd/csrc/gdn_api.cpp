// gdn_api.cpp -- C ABI of libgdn: argument checks on the host, then dispatch.
//
// Every check runs before any HIP call; a call that fails a check enqueues
// nothing.  Kernel selection is by (dtype, gate, K); V picks the number of
// 64-column blocks.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/gdn.h"
#include "chunk_bwd.h"
#include "prologue.h"

namespace gdn {
hipError_t chunk_fwd_launch(bool bf16, bool channel, int K, const void *q, const void *k,
                            const void *v, const float *g, const float *beta, const float *S0,
                            void *o, float *S_T, int B, int T, int H, int V, hipStream_t st);
hipError_t chunk_fwd_dg_launch(bool bf16, bool channel, int K, const void *q, const void *k,
                               const void *v, const float *g, const float *erase,
                               const float *write, const float *S0, void *o, float *S_T, int B,
                               int T, int H, int V, hipStream_t st);
hipError_t recurrent_step_launch(bool bf16, bool channel, int K, int V, const void *q,
                                 const void *k, const void *v, const float *g,
                                 const float *beta, const float *wg, float *S, void *o,
                                 long nslices, hipStream_t st);
hipError_t chunk_fwd_pro_launch(bool bf16, bool channel, bool silu, int K, const PrArgs &p,
                                const float *S0, void *o, float *S_T, int V, hipStream_t st);
int chunk_fwd_seg_count(long B, long T, long H);
unsigned long long chunk_fwd_seg_workspace(long B, long H, int nseg, bool want_o);
hipError_t chunk_fwd_seg_launch(const void *q, const void *k, const void *v, const float *g,
                                const float *beta, const float *S0, void *o, float *S_T, void *ws,
                                int B, int T, int H, int nseg, hipStream_t st);
unsigned long long chunk_fwd_seg_scratch_bytes();
hipError_t seg_scratch(void **p);
hipError_t recurrent_multi_launch(bool bf16, bool channel, int K, int V, const void *q,
                                  const void *k, const void *v, const float *g,
                                  const float *beta, const float *S0, void *o, float *S_T,
                                  float *S_hist, long nslices, int M, int H, hipStream_t st);
} // namespace gdn

namespace {

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
};

bool aligned(const void *p, unsigned a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1u)) == 0; }
bool aligned16(const void *p) { return aligned(p, 16); }

Range range(const void *p, unsigned long long bytes) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return {lo, lo + (uintptr_t)bytes};
}

bool overlap(Range a, Range b) {
    if (a.lo == a.hi || b.lo == b.hi) return false;
    return a.lo < b.hi && b.lo < a.hi;
}

bool kv_supported(int x) { return x == 64 || x == 128; }

// n = a * b * c * d without overflow past 2^62, or -1.
long long prod(long long a, long long b, long long c = 1, long long d = 1) {
    const long long lim = 1LL << 62;
    long long n = a;
    for (long long f : {b, c, d}) {
        if (f != 0 && n > lim / f) return -1;
        n *= f;
    }
    return n;
}

// The chunk kernels address a chunk's rows with 32-bit per-lane offsets from a
// wave-uniform base: 64 rows of H * max(K, V) elements of at most 4 bytes must
// stay below 2^31 bytes.
bool chunk_offsets_fit(long long H, int K, int V) {
    const long long w = K > V ? K : V;
    const long long n = prod(64 * 4, H, w);
    return n >= 0 && n < (1LL << 31);
}

// Argument checks of the chunkwise forward (shared by gdn_chunk_fwd and
// gdn_chunk_fwd_ws).  GDN_OK means a kernel exists for the call.
gdn_status chunk_fwd_check(const void *q, const void *k, const void *v, const float *g,
                           const float *beta, const float *S0, const void *o, const float *S_T,
                           int B, int T, int H, int K, int V, int chunk, gdn_dtype dtype,
                           gdn_gate gate)
{
    if (dtype != GDN_F32 && dtype != GDN_BF16) return GDN_EINVAL;
    if (gate != GDN_GATE_HEAD && gate != GDN_GATE_CHANNEL) return GDN_EINVAL;
    if (B < 0 || T < 0 || H < 0 || K <= 0 || V <= 0 || chunk <= 0) return GDN_EINVAL;
    if (!o && !S_T) return GDN_EINVAL;
    const long long es = dtype == GDN_BF16 ? 2 : 4;
    const long long ntok = prod(B, T, H);
    const long long nqk = prod(B, T, H, K), nv = prod(B, T, H, V), nst = prod(B, H, K, V);
    if (ntok < 0 || nqk < 0 || nv < 0 || nst < 0) return GDN_EINVAL;
    const long long ng = gate == GDN_GATE_CHANNEL ? nqk : ntok;
    if (ntok > 0 && (!q || !k || !v || !g || !beta)) return GDN_EINVAL;
    // q, k, v (and a per-channel g) are read as 16-byte vectors from row starts;
    // the rest is accessed element by element.
    for (const void *p : {q, k, v})
        if (p && !aligned16(p)) return GDN_EINVAL;
    if (g && !aligned(g, gate == GDN_GATE_CHANNEL ? 16 : 4)) return GDN_EINVAL;
    for (const void *p : {(const void *)beta, (const void *)S0, (const void *)S_T})
        if (p && !aligned(p, 4)) return GDN_EINVAL;
    if (o && !aligned16(o)) return GDN_EINVAL;   // written as 16-byte row pieces
    // o must not touch any input or the state; S_T may be S0 exactly.
    const Range rq = range(q, nqk * es), rk = range(k, nqk * es), rv = range(v, nv * es);
    const Range rg = range(g, ng * 4), rb = range(beta, ntok * 4);
    const Range rs0 = range(S0, S0 ? nst * 4 : 0), rst = range(S_T, S_T ? nst * 4 : 0);
    const Range ro = range(o, o ? nv * es : 0);
    for (Range r : {rq, rk, rv, rg, rb, rs0, rst})
        if (overlap(ro, r)) return GDN_EINVAL;
    for (Range r : {rq, rk, rv, rg, rb})
        if (overlap(rst, r)) return GDN_EINVAL;
    if (S0 && S_T && (const void *)S0 != (const void *)S_T && overlap(rs0, rst)) return GDN_EINVAL;

    if (!kv_supported(K) || !kv_supported(V) || chunk != 64) return GDN_ENOTSUP;
    if (dtype == GDN_F32 && K != 64) return GDN_ENOTSUP;
    if (prod(B, H, V / 64) > 0x7fffffffLL) return GDN_ENOTSUP;
    if (!chunk_offsets_fit(H, K, V)) return GDN_ENOTSUP;
    return GDN_OK;
}

// Segments of the sequence-parallel form for a chunkwise forward (1: the
// sequential kernels) and the workspace it needs.  Calls with bf16 operands,
// the per-key-channel gate and K = V = 128 take that form (with_o: also those
// that write o; the entry point that allocates nothing plans final-state calls
// only).
int chunk_fwd_plan(int B, int T, int H, int K, int V, gdn_dtype dtype, gdn_gate gate, bool want_o,
                   unsigned long long *bytes, bool with_o = true)
{
    *bytes = 0;
    if ((want_o && !with_o) || dtype != GDN_BF16 || gate != GDN_GATE_CHANNEL || K != 128 || V != 128)
        return 1;
    const int nseg = gdn::chunk_fwd_seg_count(B, T, H);
    *bytes = gdn::chunk_fwd_seg_workspace(B, H, nseg, want_o);
    return nseg;
}

// Size checks shared by gdn_chunk_bwd and its workspace query: EINVAL for
// negative or overflowing sizes, ENOTSUP for shapes without a kernel or grids
// past the launch limits; *nch = number of 64-token chunks over all slices.
gdn_status bwd_sizes(int B, int T, int H, int K, int V, int chunk, long long *nch) {
    if (B < 0 || T < 0 || H < 0 || K <= 0 || V <= 0 || chunk <= 0) return GDN_EINVAL;
    const long long nqk = prod(B, T, H, K), nv = prod(B, T, H, V), nst = prod(B, H, K, V);
    if (nqk < 0 || nv < 0 || nst < 0) return GDN_EINVAL;
    if (!kv_supported(K) || !kv_supported(V) || chunk != 64) return GDN_ENOTSUP;
    if (!chunk_offsets_fit(H, K, V)) return GDN_ENOTSUP;
    const long long n = prod(B, H, (T + 63) / 64);
    const long long nvb = prod(B, H, V / gdn::BW_VB);
    // one workgroup of at most 512 threads per chunk, of 256 per value block:
    // grid x * threads < 2^32
    if (n < 0 || nvb < 0 || n >= (1LL << 23) || nvb >= (1LL << 24)) return GDN_ENOTSUP;
    *nch = n;
    return GDN_OK;
}

} // namespace

extern "C" {

const char *gdn_status_str(gdn_status s) {
    switch (s) {
    case GDN_OK: return "ok";
    case GDN_EINVAL: return "invalid argument";
    case GDN_ENOTSUP: return "unsupported shape or type";
    case GDN_EHIP: return "HIP launch failed";
    }
    return "unknown status";
}

int gdn_abi_version(void) { return GDN_ABI_VERSION; }

gdn_status gdn_chunk_fwd(const void *q, const void *k, const void *v, const float *g,
                         const float *beta, const float *S0, void *o, float *S_T,
                         int B, int T, int H, int K, int V, int chunk,
                         gdn_dtype dtype, gdn_gate gate, void *stream)
{
    const gdn_status st = chunk_fwd_check(q, k, v, g, beta, S0, o, S_T, B, T, H, K, V, chunk,
                                          dtype, gate);
    if (st != GDN_OK) return st;
    if (B == 0 || H == 0) return GDN_OK;
    if (!S_T && T == 0) return GDN_OK;  // nothing to write

    const hipError_t e = gdn::chunk_fwd_launch(dtype == GDN_BF16, gate == GDN_GATE_CHANNEL, K,
                                               q, k, v, g, beta, S0, o, S_T, B, T, H, V,
                                               static_cast<hipStream_t>(stream));
    return e == hipSuccess ? GDN_OK : GDN_EHIP;
}

gdn_status gdn_chunk_fwd_workspace_size(int B, int T, int H, int K, int V, int chunk,
                                        gdn_dtype dtype, gdn_gate gate, int want_o,
                                        size_t *bytes)
{
    if (!bytes) return GDN_EINVAL;
    if (dtype != GDN_F32 && dtype != GDN_BF16) return GDN_EINVAL;
    if (gate != GDN_GATE_HEAD && gate != GDN_GATE_CHANNEL) return GDN_EINVAL;
    if (B < 0 || T < 0 || H < 0 || K <= 0 || V <= 0 || chunk <= 0) return GDN_EINVAL;
    if (prod(B, T, H, K > V ? K : V) < 0) return GDN_EINVAL;
    if (!kv_supported(K) || !kv_supported(V) || chunk != 64) return GDN_ENOTSUP;
    if (dtype == GDN_F32 && K != 64) return GDN_ENOTSUP;
    if (prod(B, H, V / 64) > 0x7fffffffLL || !chunk_offsets_fit(H, K, V)) return GDN_ENOTSUP;
    unsigned long long need = 0;
    chunk_fwd_plan(B, T, H, K, V, dtype, gate, want_o != 0, &need);
    *bytes = (size_t)need;
    return GDN_OK;
}

gdn_status gdn_chunk_fwd_ws(const void *q, const void *k, const void *v, const float *g,
                            const float *beta, const float *S0, void *o, float *S_T,
                            void *workspace, size_t workspace_bytes,
                            int B, int T, int H, int K, int V, int chunk,
                            gdn_dtype dtype, gdn_gate gate, void *stream)
{
    const gdn_status st = chunk_fwd_check(q, k, v, g, beta, S0, o, S_T, B, T, H, K, V, chunk,
                                          dtype, gate);
    if (st != GDN_OK) return st;
    unsigned long long need = 0;
    int nseg = chunk_fwd_plan(B, T, H, K, V, dtype, gate, o != nullptr, &need);
    if (need > 0) {
        if (!workspace || !aligned(workspace, 256) || workspace_bytes < need) return GDN_EINVAL;
        // the workspace must not touch any input or output
        const long long es = dtype == GDN_BF16 ? 2 : 4;
        const long long nqk = prod(B, T, H, K), nv = prod(B, T, H, V), nst = prod(B, H, K, V);
        const long long ng = gate == GDN_GATE_CHANNEL ? nqk : prod(B, T, H);
        const Range rw = range(workspace, need);
        const Range all[] = {range(q, nqk * es), range(k, nqk * es), range(v, nv * es),
                             range(g, ng * 4), range(beta, prod(B, T, H) * 4),
                             range(S0, S0 ? nst * 4 : 0), range(S_T, S_T ? nst * 4 : 0),
                             range(o, o ? nv * es : 0)};
        for (Range r : all)
            if (overlap(rw, r)) return GDN_EINVAL;
    }
    if (B == 0 || H == 0) return GDN_OK;
    if (!S_T && T == 0) return GDN_OK;
    // The o pass starts segment 0 from S0 after the final state is written:
    // with S_T in place over S0 (or no S_T at all) the call runs sequentially.
    if (o && (!S_T || (S0 && (const void *)S0 == (const void *)S_T))) nseg = 1;
    hipError_t e;
    if (nseg > 1)
        e = gdn::chunk_fwd_seg_launch(q, k, v, g, beta, S0, o, S_T, workspace, B, T, H, nseg,
                                      static_cast<hipStream_t>(stream));
    else
        e = gdn::chunk_fwd_launch(dtype == GDN_BF16, gate == GDN_GATE_CHANNEL, K, q, k, v, g, beta,
                                  S0, o, S_T, B, T, H, V, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? GDN_OK : GDN_EHIP;
}

gdn_status gdn_chunk_fwd_noalloc(const void *q, const void *k, const void *v, const float *g,
                                 const float *beta, const float *S0, void *o, float *S_T,
                                 int B, int T, int H, int K, int V, int chunk,
                                 gdn_dtype dtype, gdn_gate gate, void *stream)
{
    const gdn_status st = chunk_fwd_check(q, k, v, g, beta, S0, o, S_T, B, T, H, K, V, chunk,
                                          dtype, gate);
    if (st != GDN_OK) return st;
    unsigned long long need = 0;
    const int nseg = chunk_fwd_plan(B, T, H, K, V, dtype, gate, o != nullptr, &need, false);
    // the segment maps must fit the library's static scratch
    if (need > gdn::chunk_fwd_seg_scratch_bytes()) return GDN_ENOTSUP;
    if (B == 0 || H == 0) return GDN_OK;
    if (!S_T && T == 0) return GDN_OK;
    hipError_t e;
    if (nseg > 1) {
        void *ws = nullptr;
        e = gdn::seg_scratch(&ws);
        if (e == hipSuccess)
            e = gdn::chunk_fwd_seg_launch(nullptr, k, v, g, beta, S0, nullptr, S_T, ws, B, T, H,
                                          nseg, static_cast<hipStream_t>(stream));
    } else {
        e = gdn::chunk_fwd_launch(dtype == GDN_BF16, gate == GDN_GATE_CHANNEL, K, q, k, v, g, beta,
                                  S0, o, S_T, B, T, H, V, static_cast<hipStream_t>(stream));
    }
    return e == hipSuccess ? GDN_OK : GDN_EHIP;
}

} // extern "C"

namespace {

// Checks and launch of one decode step; wg is the decoupled write gate or
// nullptr (beta writes too).
gdn_status recurrent_step_impl(const void *q, const void *k, const void *v, const float *g,
                               const float *beta, const float *wg, bool need_wg, float *S,
                               void *o, int N, int H, int K, int V, gdn_dtype dtype,
                               gdn_gate gate, void *stream)
{
    if (dtype != GDN_F32 && dtype != GDN_BF16) return GDN_EINVAL;
    if (gate != GDN_GATE_HEAD && gate != GDN_GATE_CHANNEL) return GDN_EINVAL;
    if (N < 0 || H < 0 || K <= 0 || V <= 0) return GDN_EINVAL;
    const long long es = dtype == GDN_BF16 ? 2 : 4;
    const long long ns = prod(N, H), nqk = prod(N, H, K), nv = prod(N, H, V), nst = prod(N, H, K, V);
    if (ns < 0 || nqk < 0 || nv < 0 || nst < 0) return GDN_EINVAL;
    const long long ng = gate == GDN_GATE_CHANNEL ? nqk : ns;
    if (ns > 0 && (!q || !k || !v || !g || !beta || !S)) return GDN_EINVAL;
    if (ns > 0 && need_wg && !wg) return GDN_EINVAL;
    // The state is streamed as 16-byte vectors; the vectors are read per element.
    if (S && !aligned16(S)) return GDN_EINVAL;
    for (const void *p : {q, k, v, (const void *)o})
        if (p && !aligned(p, (unsigned)es)) return GDN_EINVAL;
    for (const void *p : {(const void *)g, (const void *)beta, (const void *)wg})
        if (p && !aligned(p, 4)) return GDN_EINVAL;
    const Range rq = range(q, nqk * es), rk = range(k, nqk * es), rv = range(v, nv * es);
    const Range rg = range(g, ng * 4), rb = range(beta, ns * 4), rs = range(S, nst * 4);
    const Range rw = range(wg, wg ? ns * 4 : 0);
    const Range ro = range(o, o ? nv * es : 0);
    for (Range r : {rq, rk, rv, rg, rb, rw, rs})
        if (overlap(ro, r)) return GDN_EINVAL;
    for (Range r : {rq, rk, rv, rg, rb, rw})
        if (overlap(rs, r)) return GDN_EINVAL;

    if (!kv_supported(K) || !kv_supported(V)) return GDN_ENOTSUP;
    if (ns > 0x7fffffffLL) return GDN_ENOTSUP;
    if (ns == 0) return GDN_OK;

    const hipError_t e = gdn::recurrent_step_launch(dtype == GDN_BF16, gate == GDN_GATE_CHANNEL,
                                                    K, V, q, k, v, g, beta, wg, S, o, ns,
                                                    static_cast<hipStream_t>(stream));
    return e == hipSuccess ? GDN_OK : GDN_EHIP;
}

} // namespace

extern "C" {

gdn_status gdn_recurrent_step(const void *q, const void *k, const void *v, const float *g,
                              const float *beta, float *S, void *o, int N, int H, int K,
                              int V, gdn_dtype dtype, gdn_gate gate, void *stream)
{
    return recurrent_step_impl(q, k, v, g, beta, nullptr, false, S, o, N, H, K, V, dtype, gate,
                               stream);
}

gdn_status gdn_recurrent_step_decoupled(const void *q, const void *k, const void *v,
                                        const float *g, const float *erase, const float *write,
                                        float *S, void *o, int N, int H, int K, int V,
                                        gdn_dtype dtype, gdn_gate gate, void *stream)
{
    return recurrent_step_impl(q, k, v, g, erase, write, true, S, o, N, H, K, V, dtype, gate,
                               stream);
}

gdn_status gdn_chunk_fwd_decoupled(const void *q, const void *k, const void *v, const float *g,
                                   const float *erase, const float *write, const float *S0,
                                   void *o, float *S_T, int B, int T, int H, int K, int V,
                                   int chunk, gdn_dtype dtype, gdn_gate gate, void *stream)
{
    const gdn_status st = chunk_fwd_check(q, k, v, g, erase, S0, o, S_T, B, T, H, K, V, chunk,
                                          dtype, gate);
    if (st != GDN_OK) return st;
    const long long ntok = prod(B, T, H);
    if (ntok > 0 && !write) return GDN_EINVAL;
    if (write && !aligned(write, 4)) return GDN_EINVAL;
    const Range rw = range(write, write ? ntok * 4 : 0);
    const long long es = dtype == GDN_BF16 ? 2 : 4;
    if (o && overlap(range(o, prod(B, T, H, V) * es), rw)) return GDN_EINVAL;
    if (S_T && overlap(range(S_T, prod(B, H, K, V) * 4), rw)) return GDN_EINVAL;
    if (B == 0 || H == 0) return GDN_OK;
    if (!S_T && T == 0) return GDN_OK;
    const hipError_t e = gdn::chunk_fwd_dg_launch(dtype == GDN_BF16, gate == GDN_GATE_CHANNEL, K,
                                                  q, k, v, g, erase, write, S0, o, S_T, B, T, H,
                                                  V, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? GDN_OK : GDN_EHIP;
}

gdn_status gdn_recurrent_steps(const void *q, const void *k, const void *v, const float *g,
                               const float *beta, const float *S0, void *o, float *S_T,
                               float *S_hist, int N, int M, int H, int K, int V,
                               gdn_dtype dtype, gdn_gate gate, void *stream)
{
    if (dtype != GDN_F32 && dtype != GDN_BF16) return GDN_EINVAL;
    if (gate != GDN_GATE_HEAD && gate != GDN_GATE_CHANNEL) return GDN_EINVAL;
    if (N < 0 || M < 0 || H < 0 || K <= 0 || V <= 0) return GDN_EINVAL;
    if (!o && !S_T && !S_hist) return GDN_EINVAL;
    const long long es = dtype == GDN_BF16 ? 2 : 4;
    const long long ns = prod(N, H), ntok = prod(N, M, H);
    const long long nqk = prod(N, M, H, K), nv = prod(N, M, H, V), nst = prod(N, H, K, V);
    const long long nhist = nqk < 0 ? -1 : prod(nqk, V);
    if (ns < 0 || ntok < 0 || nqk < 0 || nv < 0 || nst < 0 || nhist < 0) return GDN_EINVAL;
    const long long ng = gate == GDN_GATE_CHANNEL ? nqk : ntok;
    if (ntok > 0 && (!q || !k || !v || !g || !beta)) return GDN_EINVAL;
    // The vectors are read and o written element by element; every state tensor
    // is streamed as 16-byte vectors.
    for (const void *p : {q, k, v, (const void *)o})
        if (p && !aligned(p, (unsigned)es)) return GDN_EINVAL;
    for (const void *p : {(const void *)g, (const void *)beta})
        if (p && !aligned(p, 4)) return GDN_EINVAL;
    for (const void *p : {(const void *)S0, (const void *)S_T, (const void *)S_hist})
        if (p && !aligned16(p)) return GDN_EINVAL;
    // No output may touch an input or another output; S_T may be S0 exactly.
    const Range rq = range(q, nqk * es), rk = range(k, nqk * es), rv = range(v, nv * es);
    const Range rg = range(g, ng * 4), rb = range(beta, ntok * 4);
    const Range rs0 = range(S0, S0 ? nst * 4 : 0), rst = range(S_T, S_T ? nst * 4 : 0);
    const Range ro = range(o, o ? nv * es : 0), rh = range(S_hist, S_hist ? nhist * 4 : 0);
    for (Range r : {rq, rk, rv, rg, rb, rs0, rst, rh})
        if (overlap(ro, r)) return GDN_EINVAL;
    for (Range r : {rq, rk, rv, rg, rb, rs0, rst})
        if (overlap(rh, r)) return GDN_EINVAL;
    for (Range r : {rq, rk, rv, rg, rb})
        if (overlap(rst, r)) return GDN_EINVAL;
    if (S0 && S_T && (const void *)S0 != (const void *)S_T && overlap(rs0, rst)) return GDN_EINVAL;

    if (!kv_supported(K) || !kv_supported(V)) return GDN_ENOTSUP;
    if (prod(ns, V / 64 > 0 ? V / 64 : 1) > 0x7fffffffLL) return GDN_ENOTSUP;
    if (ns == 0) return GDN_OK;
    if (M == 0 && !S_T) return GDN_OK;   // nothing to write

    const hipError_t e = gdn::recurrent_multi_launch(dtype == GDN_BF16, gate == GDN_GATE_CHANNEL,
                                                     K, V, q, k, v, g, beta, S0, o, S_T, S_hist,
                                                     ns, M, H, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? GDN_OK : GDN_EHIP;
}

gdn_status gdn_chunk_bwd_workspace_size(int B, int T, int H, int K, int V, int chunk,
                                        size_t *bytes)
{
    if (!bytes) return GDN_EINVAL;
    long long nch = 0;
    const gdn_status st = bwd_sizes(B, T, H, K, V, chunk, &nch);
    if (st != GDN_OK) return st;
    *bytes = (size_t)gdn::bw_workspace((unsigned long long)nch, K, V, nullptr, nullptr);
    return GDN_OK;
}

gdn_status gdn_chunk_bwd(const void *q, const void *k, const void *v, const float *g,
                         const float *beta, const float *S0, const void *d_o, const float *dS_T,
                         void *dq, void *dk, void *dv, float *dg, float *dbeta, float *dS0,
                         void *workspace, size_t workspace_bytes, int B, int T, int H, int K,
                         int V, int chunk, gdn_dtype dtype, gdn_gate gate, void *stream)
{
    if (dtype != GDN_F32 && dtype != GDN_BF16) return GDN_EINVAL;
    if (gate != GDN_GATE_HEAD && gate != GDN_GATE_CHANNEL) return GDN_EINVAL;
    if (B < 0 || T < 0 || H < 0 || K <= 0 || V <= 0 || chunk <= 0) return GDN_EINVAL;
    const long long es = dtype == GDN_BF16 ? 2 : 4;
    const long long ntok = prod(B, T, H);
    const long long nqk = prod(B, T, H, K), nv = prod(B, T, H, V), nst = prod(B, H, K, V);
    if (ntok < 0 || nqk < 0 || nv < 0 || nst < 0) return GDN_EINVAL;
    const long long ng = gate == GDN_GATE_CHANNEL ? nqk : ntok;
    if (ntok > 0 && (!q || !k || !v || !g || !beta || !d_o || !dq || !dk || !dv || !dg || !dbeta))
        return GDN_EINVAL;
    // q, k, v, d_o, a per-channel g, S0 and dS_T are read as 16-byte vectors
    // from row starts; the outputs are written element by element.
    for (const void *p : {q, k, v, d_o, (const void *)S0, (const void *)dS_T})
        if (p && !aligned16(p)) return GDN_EINVAL;
    if (g && !aligned(g, gate == GDN_GATE_CHANNEL ? 16 : 4)) return GDN_EINVAL;
    for (const void *p : {(const void *)dq, (const void *)dk, (const void *)dv})
        if (p && !aligned(p, (unsigned)es)) return GDN_EINVAL;
    for (const void *p : {(const void *)beta, (const void *)dg, (const void *)dbeta,
                          (const void *)dS0})
        if (p && !aligned(p, 4)) return GDN_EINVAL;
    if (workspace && !aligned(workspace, 256)) return GDN_EINVAL;

    long long nch = 0;
    const gdn_status st = bwd_sizes(B, T, H, K, V, chunk, &nch);
    if (st == GDN_EINVAL) return st;
    // the workspace check needs the size, which needs a supported shape
    const unsigned long long need =
        st == GDN_OK ? gdn::bw_workspace((unsigned long long)nch, K, V, nullptr, nullptr) : 0;
    if (need > 0 && (!workspace || workspace_bytes < need)) return GDN_EINVAL;

    // No output may touch an input, another output or the workspace.
    const Range in[] = {range(q, nqk * es), range(k, nqk * es), range(v, nv * es),
                        range(g, ng * 4), range(beta, ntok * 4), range(S0, S0 ? nst * 4 : 0),
                        range(d_o, nv * es), range(dS_T, dS_T ? nst * 4 : 0)};
    const Range out[] = {range(dq, nqk * es), range(dk, nqk * es), range(dv, nv * es),
                         range(dg, ng * 4), range(dbeta, ntok * 4),
                         range(dS0, dS0 ? nst * 4 : 0), range(workspace, need)};
    const int nout = sizeof(out) / sizeof(out[0]);
    for (int i = 0; i < nout; ++i) {
        for (Range r : in)
            if (overlap(out[i], r)) return GDN_EINVAL;
        for (int j = i + 1; j < nout; ++j)
            if (overlap(out[i], out[j])) return GDN_EINVAL;
    }
    if (st != GDN_OK) return st;   // ENOTSUP
    if (B == 0 || H == 0) return GDN_OK;
    if (T == 0 && !dS0) return GDN_OK;   // nothing to write

    gdn::BwArgs a;
    a.q = q; a.k = k; a.v = v; a.d_o = d_o;
    a.g = g; a.beta = beta; a.S0 = S0; a.dS_T = dS_T;
    a.dq = dq; a.dk = dk; a.dv = dv;
    a.dg = dg; a.dbeta = dbeta; a.dS0 = dS0;
    gdn::bw_workspace((unsigned long long)nch, K, V, workspace, &a.ws);
    a.T = T; a.H = H; a.NC = (T + 63) / 64; a.NS = B * H;
    const hipError_t e = gdn::chunk_bwd_launch(dtype == GDN_BF16, gate == GDN_GATE_CHANNEL, K, V,
                                               a, (long)B * H, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? GDN_OK : GDN_EHIP;
}

gdn_status gdn_prologue(const void *q_raw, const void *k_raw, const void *v_raw, const float *g_raw,
                        const float *b_raw, const float *w_q, const float *w_k, const float *w_v,
                        const void *cs_q, const void *cs_k, const void *cs_v, void *q, void *k,
                        void *v, float *g, float *beta, void *cs_q_out, void *cs_k_out,
                        void *cs_v_out, int B, int T, int H, int K, int V, float g_cap,
                        gdn_act act, gdn_dtype dtype, gdn_gate gate, void *stream)
{
    if (dtype != GDN_F32 && dtype != GDN_BF16) return GDN_EINVAL;
    if (gate != GDN_GATE_HEAD && gate != GDN_GATE_CHANNEL) return GDN_EINVAL;
    if (act != GDN_ACT_NONE && act != GDN_ACT_SILU) return GDN_EINVAL;
    if (B < 0 || T < 0 || H < 0 || K <= 0 || V <= 0 || !(g_cap > 0.f)) return GDN_EINVAL;
    const long long es = dtype == GDN_BF16 ? 2 : 4;
    const long long ntok = prod(B, T, H), nqk = prod(B, T, H, K), nv = prod(B, T, H, V);
    const long long nsk = prod(B, 3, H, K), nsv = prod(B, 3, H, V);
    const long long nwk = prod(H, K, 4), nwv = prod(H, V, 4);
    if (ntok < 0 || nqk < 0 || nv < 0 || nsk < 0 || nsv < 0 || nwk < 0 || nwv < 0) return GDN_EINVAL;
    const bool ch = gate == GDN_GATE_CHANNEL;
    const long long ng = ch ? nqk : ntok;
    if (ntok > 0 && (!q_raw || !k_raw || !v_raw || !g_raw || !b_raw || !w_q || !w_k || !w_v ||
                     !q || !k || !v || !g || !beta))
        return GDN_EINVAL;
    for (const void *p : {q_raw, k_raw, v_raw, (const void *)q, (const void *)k, (const void *)v,
                          (const void *)w_q, (const void *)w_k, (const void *)w_v, cs_q, cs_k,
                          cs_v, (const void *)cs_q_out, (const void *)cs_k_out,
                          (const void *)cs_v_out})
        if (p && !aligned16(p)) return GDN_EINVAL;
    for (const void *p : {(const void *)g_raw, (const void *)g})
        if (p && !aligned(p, ch ? 16 : 4)) return GDN_EINVAL;
    for (const void *p : {(const void *)b_raw, (const void *)beta})
        if (p && !aligned(p, 4)) return GDN_EINVAL;
    const Range in[] = {range(q_raw, nqk * es), range(k_raw, nqk * es), range(v_raw, nv * es),
                        range(g_raw, ng * 4), range(b_raw, ntok * 4), range(w_q, nwk * 4),
                        range(w_k, nwk * 4), range(w_v, nwv * 4)};
    const Range sin[] = {range(cs_q, cs_q ? nsk * es : 0), range(cs_k, cs_k ? nsk * es : 0),
                         range(cs_v, cs_v ? nsv * es : 0)};
    const Range sout[] = {range(cs_q_out, cs_q_out ? nsk * es : 0),
                          range(cs_k_out, cs_k_out ? nsk * es : 0),
                          range(cs_v_out, cs_v_out ? nsv * es : 0)};
    const Range out[] = {range(q, nqk * es), range(k, nqk * es), range(v, nv * es),
                         range(g, ng * 4), range(beta, ntok * 4), sout[0], sout[1], sout[2]};
    const int nout = sizeof(out) / sizeof(out[0]);
    for (int i = 0; i < nout; ++i) {
        for (Range r : in)
            if (overlap(out[i], r)) return GDN_EINVAL;
        for (int j = 0; j < 3; ++j) {
            // a state output may be exactly its own input
            const bool own = i >= 5 && i - 5 == j && sin[j].lo == out[i].lo && sin[j].hi == out[i].hi;
            if (!own && overlap(out[i], sin[j])) return GDN_EINVAL;
        }
        for (int j = i + 1; j < nout; ++j)
            if (overlap(out[i], out[j])) return GDN_EINVAL;
    }
    if (!kv_supported(K) || !kv_supported(V)) return GDN_ENOTSUP;
    // the per-channel chunk kernels split the decay at 16-token blocks, which
    // keeps every factor in range for g >= -5 only: a larger cap would produce
    // inputs they cannot take
    if (ch && !(g_cap <= 5.f)) return GDN_ENOTSUP;
    // one thread per token and 8 channels (at most 16 per token): the grid's
    // work-items must stay below 2^32
    if (prod(ntok, 16) >= (1LL << 32) || prod(B, H, 16) >= (1LL << 32)) return GDN_ENOTSUP;
    if (B == 0 || H == 0) return GDN_OK;
    if (T == 0 && !cs_q_out && !cs_k_out && !cs_v_out) return GDN_OK;

    gdn::PrArgs a;
    a.q_raw = q_raw; a.k_raw = k_raw; a.v_raw = v_raw; a.g_raw = g_raw; a.b_raw = b_raw;
    a.w_q = w_q; a.w_k = w_k; a.w_v = w_v; a.cs_q = cs_q; a.cs_k = cs_k; a.cs_v = cs_v;
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta;
    a.cs_q_out = cs_q_out; a.cs_k_out = cs_k_out; a.cs_v_out = cs_v_out;
    a.cap = g_cap; a.B = B; a.T = T; a.H = H;
    const hipError_t e = gdn::prologue_launch(dtype == GDN_BF16, ch, act == GDN_ACT_SILU, K, V, a,
                                              static_cast<hipStream_t>(stream));
    return e == hipSuccess ? GDN_OK : GDN_EHIP;
}

gdn_status gdn_chunk_fwd_prologue(const void *q_raw, const void *k_raw, const void *v_raw,
                                  const float *g_raw, const float *b_raw, const float *w_q,
                                  const float *w_k, const float *w_v, const void *cs_q,
                                  const void *cs_k, const void *cs_v, void *cs_q_out,
                                  void *cs_k_out, void *cs_v_out, const float *S0, void *o,
                                  float *S_T, int B, int T, int H, int K, int V, int chunk,
                                  float g_cap, gdn_act act, gdn_dtype dtype, gdn_gate gate,
                                  void *stream)
{
    // the chunkwise forward's own checks, with the raw projections in place of
    // q, k, v, g and beta (same shapes and alignment)
    const gdn_status st = chunk_fwd_check(q_raw, k_raw, v_raw, g_raw, b_raw, S0, o, S_T, B, T, H,
                                          K, V, chunk, dtype, gate);
    if (st != GDN_OK) return st;
    if (act != GDN_ACT_NONE && act != GDN_ACT_SILU) return GDN_EINVAL;
    if (!(g_cap > 0.f)) return GDN_EINVAL;
    const long long es = dtype == GDN_BF16 ? 2 : 4;
    const long long ntok = prod(B, T, H), nqk = prod(B, T, H, K), nv = prod(B, T, H, V);
    const long long nsk = prod(B, 3, H, K), nsv = prod(B, 3, H, V);
    const long long nwk = prod(H, K, 4), nwv = prod(H, V, 4);
    if (nsk < 0 || nsv < 0 || nwk < 0 || nwv < 0) return GDN_EINVAL;
    const bool ch = gate == GDN_GATE_CHANNEL;
    if (B > 0 && H > 0 && (!w_q || !w_k || !w_v)) return GDN_EINVAL;
    for (const void *p : {(const void *)w_q, (const void *)w_k, (const void *)w_v, cs_q, cs_k, cs_v,
                          (const void *)cs_q_out, (const void *)cs_k_out, (const void *)cs_v_out})
        if (p && !aligned16(p)) return GDN_EINVAL;
    const Range in[] = {range(q_raw, nqk * es), range(k_raw, nqk * es), range(v_raw, nv * es),
                        range(g_raw, (ch ? nqk : ntok) * 4), range(b_raw, ntok * 4),
                        range(w_q, nwk * 4), range(w_k, nwk * 4), range(w_v, nwv * 4),
                        range(cs_q, cs_q ? nsk * es : 0), range(cs_k, cs_k ? nsk * es : 0),
                        range(cs_v, cs_v ? nsv * es : 0), range(S0, S0 ? prod(B, H, K, V) * 4 : 0)};
    // every output apart from S_T (which may be S0) touches no input and no other
    // output; a carried state out is never its own input here, since each
    // column block of a head reads the incoming state while another may be
    // writing the outgoing one
    const Range out[] = {range(cs_q_out, cs_q_out ? nsk * es : 0),
                         range(cs_k_out, cs_k_out ? nsk * es : 0),
                         range(cs_v_out, cs_v_out ? nsv * es : 0),
                         range(o, o ? nv * es : 0), range(S_T, S_T ? prod(B, H, K, V) * 4 : 0)};
    for (int i = 0; i < 5; ++i) {
        for (int j = 0; j < (int)(sizeof(in) / sizeof(in[0])); ++j) {
            if (i == 4 && j == 11 && (const void *)S0 == (const void *)S_T) continue;
            if (overlap(out[i], in[j])) return GDN_EINVAL;
        }
        for (int j = i + 1; j < 5; ++j)
            if (overlap(out[i], out[j])) return GDN_EINVAL;
    }
    // the per-channel chunk kernels take g >= -5 only (the 16-token decay split)
    if (ch && !(g_cap <= 5.f)) return GDN_ENOTSUP;
    if (B == 0 || H == 0) return GDN_OK;
    if (!S_T && T == 0 && !cs_q_out && !cs_k_out && !cs_v_out) return GDN_OK;

    gdn::PrArgs p = {};
    p.q_raw = q_raw; p.k_raw = k_raw; p.v_raw = v_raw; p.g_raw = g_raw; p.b_raw = b_raw;
    p.w_q = w_q; p.w_k = w_k; p.w_v = w_v; p.cs_q = cs_q; p.cs_k = cs_k; p.cs_v = cs_v;
    p.cs_q_out = cs_q_out; p.cs_k_out = cs_k_out; p.cs_v_out = cs_v_out;
    p.cap = g_cap; p.B = B; p.T = T; p.H = H;
    const hipError_t e = gdn::chunk_fwd_pro_launch(dtype == GDN_BF16, ch, act == GDN_ACT_SILU, K, p,
                                                   S0, o, S_T, V, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? GDN_OK : GDN_EHIP;
}

gdn_status gdn_recurrent_step_prologue(const void *q_raw, const void *k_raw, const void *v_raw,
                                       const float *g_raw, const float *b_raw, const float *w_q,
                                       const float *w_k, const float *w_v, const void *cs_q,
                                       const void *cs_k, const void *cs_v, void *cs_q_out,
                                       void *cs_k_out, void *cs_v_out, float *S, void *o, int N,
                                       int H, int K, int V, float g_cap, gdn_act act,
                                       gdn_dtype dtype, gdn_gate gate, void *stream)
{
    if (dtype != GDN_F32 && dtype != GDN_BF16) return GDN_EINVAL;
    if (gate != GDN_GATE_HEAD && gate != GDN_GATE_CHANNEL) return GDN_EINVAL;
    if (act != GDN_ACT_NONE && act != GDN_ACT_SILU) return GDN_EINVAL;
    if (N < 0 || H < 0 || K <= 0 || V <= 0 || !(g_cap > 0.f)) return GDN_EINVAL;
    const long long es = dtype == GDN_BF16 ? 2 : 4;
    const long long ns = prod(N, H), nk = prod(N, H, K), nv = prod(N, H, V);
    const long long nsk = prod(N, 3, H, K), nsv = prod(N, 3, H, V), nst = prod(N, H, K, V);
    const long long nwk = prod(H, K, 4), nwv = prod(H, V, 4);
    if (ns < 0 || nk < 0 || nv < 0 || nsk < 0 || nsv < 0 || nst < 0 || nwk < 0 || nwv < 0)
        return GDN_EINVAL;
    const bool ch = gate == GDN_GATE_CHANNEL;
    const long long ng = ch ? nk : ns;
    if (ns > 0 && (!q_raw || !k_raw || !v_raw || !g_raw || !b_raw || !w_q || !w_k || !w_v || !S))
        return GDN_EINVAL;
    for (const void *p : {q_raw, k_raw, v_raw, cs_q, cs_k, cs_v, (const void *)cs_q_out,
                          (const void *)cs_k_out, (const void *)cs_v_out, (const void *)o})
        if (p && !aligned(p, (unsigned)es)) return GDN_EINVAL;
    for (const void *p : {(const void *)w_q, (const void *)w_k, (const void *)w_v, (const void *)S})
        if (p && !aligned16(p)) return GDN_EINVAL;
    for (const void *p : {(const void *)g_raw, (const void *)b_raw})
        if (p && !aligned(p, 4)) return GDN_EINVAL;
    const Range in[] = {range(q_raw, nk * es), range(k_raw, nk * es), range(v_raw, nv * es),
                        range(g_raw, ng * 4), range(b_raw, ns * 4), range(w_q, nwk * 4),
                        range(w_k, nwk * 4), range(w_v, nwv * 4),
                        range(cs_q, cs_q ? nsk * es : 0), range(cs_k, cs_k ? nsk * es : 0),
                        range(cs_v, cs_v ? nsv * es : 0)};
    const Range out[] = {range(S, nst * 4), range(o, o ? nv * es : 0),
                         range(cs_q_out, cs_q_out ? nsk * es : 0),
                         range(cs_k_out, cs_k_out ? nsk * es : 0),
                         range(cs_v_out, cs_v_out ? nsv * es : 0)};
    const int nout = sizeof(out) / sizeof(out[0]);
    for (int i = 0; i < nout; ++i) {
        for (Range r : in)
            if (overlap(out[i], r)) return GDN_EINVAL;
        for (int j = i + 1; j < nout; ++j)
            if (overlap(out[i], out[j])) return GDN_EINVAL;
    }
    if (!kv_supported(K) || !kv_supported(V)) return GDN_ENOTSUP;
    if (prod(ns, V / 64 > 0 ? V / 64 : 1) > 0x7fffffffLL) return GDN_ENOTSUP;
    if (ns == 0) return GDN_OK;

    gdn::RpArgs a;
    a.q_raw = q_raw; a.k_raw = k_raw; a.v_raw = v_raw; a.g_raw = g_raw; a.b_raw = b_raw;
    a.w_q = w_q; a.w_k = w_k; a.w_v = w_v; a.cs_q = cs_q; a.cs_k = cs_k; a.cs_v = cs_v;
    a.cs_q_out = cs_q_out; a.cs_k_out = cs_k_out; a.cs_v_out = cs_v_out;
    a.S = S; a.o = o; a.cap = g_cap; a.H = H;
    const hipError_t e = gdn::step_prologue_launch(dtype == GDN_BF16, ch, act == GDN_ACT_SILU, K, V,
                                                   a, ns, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? GDN_OK : GDN_EHIP;
}

} // extern "C"
