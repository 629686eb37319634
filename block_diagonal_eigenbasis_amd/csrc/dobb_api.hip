// C ABI of libdobb: host-side validation, workspace sizing, grouping of matrix sets by shape, and
// the optional kernel timer.  Every computation is done by the kernels in k_*.hip.
#include <map>
#include <mutex>
#include <string>
#include <tuple>
#include <vector>

#include "dobb_internal.h"

namespace dobb {

// ---- kernel timer ----------------------------------------------------------------------------
namespace {
struct Pending {
    const char *name;
    hipEvent_t a, b;
};
struct ProfState {
    bool on = false;
    const char *cur_name = nullptr;
    hipEvent_t cur = nullptr;
    std::vector<Pending> pending;
    std::vector<hipEvent_t> pool;                                   // recycled events
    std::vector<std::tuple<const char *, int64_t, double>> totals;  // name, launches, ms
};
ProfState &prof() {
    static ProfState p;
    return p;
}
hipEvent_t prof_event() {
    ProfState &p = prof();
    if (!p.pool.empty()) {
        hipEvent_t e = p.pool.back();
        p.pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}
void prof_collect() {
    ProfState &p = prof();
    for (Pending &e : p.pending) {
        float ms = 0.f;
        if (hipEventSynchronize(e.b) == hipSuccess && hipEventElapsedTime(&ms, e.a, e.b) == hipSuccess) {
            bool found = false;
            for (auto &t : p.totals)
                if (std::string(std::get<0>(t)) == e.name) { std::get<1>(t) += 1; std::get<2>(t) += ms; found = true; break; }
            if (!found) p.totals.emplace_back(e.name, 1, (double)ms);
        }
        p.pool.push_back(e.a);
        p.pool.push_back(e.b);
    }
    p.pending.clear();
}
}  // namespace

void prof_before(const char *name, hipStream_t s) {
    ProfState &p = prof();
    if (!p.on) return;
    p.cur = prof_event();
    if (!p.cur) return;
    p.cur_name = name;
    (void)hipEventRecord(p.cur, s);
}

void prof_after(hipStream_t s) {
    ProfState &p = prof();
    if (!p.on || !p.cur) return;
    hipEvent_t b = prof_event();
    if (!b) { p.pool.push_back(p.cur); p.cur = nullptr; return; }
    (void)hipEventRecord(b, s);
    p.pending.push_back({p.cur_name, p.cur, b});
    p.cur = nullptr;
    if (p.pending.size() > 4096) prof_collect();  // bound the number of live events
}

int max_lds_bytes() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 65536;
    if (!cached[dev]) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess || v <= 0) v = 65536;
        cached[dev] = v;
    }
    return cached[dev];
}

namespace {

constexpr int64_t kMaxNb = 1024;
constexpr int64_t kMaxRows = (int64_t)65535 * kBM;

inline size_t al256(size_t x) { return (x + 255) / 256 * 256; }

dobb_status check_shape(const dobb_shape *s) {
    if (!s) return DOBB_ERR_INVALID_ARG;
    if (s->m < 1 || s->n < 1 || s->nb < 1 || s->nb > kMaxNb || s->n % s->nb != 0 || s->m > kMaxRows)
        return DOBB_ERR_SHAPE;
    return DOBB_OK;
}

// Dobb-G: blocks of nb rows (m % nb == 0); the launch grid holds ceil(nb / 64) x (m / nb) tiles per
// matrix in its y dimension
dobb_status check_shape_g(const dobb_shape *s) {
    if (!s) return DOBB_ERR_INVALID_ARG;
    if (s->m < 1 || s->n < 1 || s->nb < 1 || s->nb > kMaxNb || s->m % s->nb != 0) return DOBB_ERR_SHAPE;
    if ((s->nb + kBM - 1) / kBM * (s->m / s->nb) > 65535 || (s->n + kBN - 1) / kBN > 0x7fffffff) return DOBB_ERR_SHAPE;
    return DOBB_OK;
}

// matrices per Dobb-G launch
int step_g_chunk(const dobb_shape &sh) {
    const int64_t per = (sh.nb + kBM - 1) / kBM * (sh.m / sh.nb);
    const int64_t c = 65535 / per;
    return (int)(c < kMaxMats ? c : kMaxMats);
}

bool same_shape(const dobb_shape &a, const dobb_shape &b) { return a.m == b.m && a.n == b.n && a.nb == b.nb; }

// indices of matrices grouped by identical shape, first-seen order
std::vector<std::vector<int>> group_by_shape(int count, const dobb_shape *shapes) {
    std::vector<std::vector<int>> groups;
    for (int i = 0; i < count; ++i) {
        bool placed = false;
        for (auto &g : groups)
            if (same_shape(shapes[g[0]], shapes[i])) { g.push_back(i); placed = true; break; }
        if (!placed) groups.push_back({i});
    }
    return groups;
}

size_t step_ws_one(const dobb_shape &sh, int norm) {
    if (step_bf16_eligible(sh, norm)) return step_bf16_ws_one(sh);
    const size_t mn = (size_t)sh.m * (size_t)sh.n;
    if (norm == DOBB_NORM_SIGN) return al256(mn);                 // int8 sign codes
    size_t b = al256(mn * 4) + al256((size_t)sh.n * 4);           // fp32 coefficients + column scales
    if (norm == DOBB_NORM_COL_L2)                                 // column sums of squares per 128-row tile
        b += al256((size_t)((sh.m + 127) / 128) * (size_t)sh.n * 8);
    if (norm == DOBB_NORM_COL_L2 && step_wide_eligible(sh))       // the wide kernels' basis planes
        b += al256(step_wide_planes_bytes(sh));
    return b;
}

// the fp32 copy of a bf16 basis, per matrix
size_t basis_copy_one(const dobb_shape &sh) { return al256((size_t)sh.n * (size_t)sh.nb * 4); }

size_t step_region_one(const dobb_shape &sh, int variant) {
    const bool qbf = (variant & DOBB_WS_BF16_BASIS) != 0;
    return step_ws_one(sh, variant & ~DOBB_WS_BF16_BASIS) + (qbf ? basis_copy_one(sh) : 0);
}

// Dobb-G: the step's regions, then the fp32 copy of a bf16 basis (m x nb entries)
size_t step_g_region_one(const dobb_shape &sh, int variant) {
    const bool qbf = (variant & DOBB_WS_BF16_BASIS) != 0;
    return step_g_ws_one(sh, variant & ~DOBB_WS_BF16_BASIS) + (qbf ? al256((size_t)sh.m * (size_t)sh.nb * 4) : 0);
}

size_t group_ws(dobb_op op, const dobb_shape &sh, int cnt, int64_t N, int variant) {
    const int c = cnt < kMaxMats ? cnt : kMaxMats;
    const bool qbf = (variant & DOBB_WS_BF16_BASIS) != 0;
    switch (op) {
        case DOBB_OP_STEP_G: {
            const int cg = step_g_chunk(sh);
            return step_g_region_one(sh, variant) * (cnt < cg ? cnt : cg);
        }
        case DOBB_OP_ACCUMULATE: return al256(accumulate_ws(sh, N, cnt));
        case DOBB_OP_REFRESH: return al256(refresh_ws(sh, c)) + (qbf ? basis_copy_one(sh) * c : 0);
        case DOBB_OP_STEP: return step_region_one(sh, variant) * c;
    }
    return 0;
}

dobb_status check_ws(void *ws, size_t ws_bytes, size_t need) {
    if (need == 0) return DOBB_OK;
    if (!ws || ((uintptr_t)ws & 255u) != 0 || ws_bytes < need) return DOBB_ERR_WORKSPACE;
    return DOBB_OK;
}

dobb_status hip_status(hipError_t e) { return e == hipSuccess ? DOBB_OK : DOBB_ERR_HIP; }

}  // namespace

// ---- scratch of the allocation-free step ---------------------------------------------------------
// A file-scope device array: every GPU the library is loaded on holds its own copy until the process
// ends.  Host code never uses the array's name as an address: its device address is looked up once
// per device (hipGetSymbolAddress, with that device current) and kept in scratch_ptr.  Calls on one
// GPU share the array, so calls that overlap on one GPU race.  No step kernel reads a workspace byte
// it has not written in the same call, so the array needs no clearing between calls.
static __device__ __align__(256) unsigned char scratch[DOBB_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void *scratch_ptr[kMaxDevices];

dobb_status scratch_for_current_device(void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DOBB_ERR_HIP;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return DOBB_ERR_HIP;
        scratch_ptr[dev] = p;
    }
    *out = scratch_ptr[dev];
    return DOBB_OK;
}
}  // namespace
}  // namespace dobb

using namespace dobb;

extern "C" {

int dobb_abi_version(void) { return DOBB_ABI_VERSION; }

const char *dobb_status_string(dobb_status st) {
    switch (st) {
        case DOBB_OK: return "ok";
        case DOBB_ERR_INVALID_ARG: return "invalid argument";
        case DOBB_ERR_SHAPE: return "invalid shape (need m, n, nb >= 1, n % nb == 0, nb <= 1024, ldx >= n)";
        case DOBB_ERR_DTYPE: return "unsupported dtype";
        case DOBB_ERR_WORKSPACE: return "workspace missing, misaligned (256 B) or too small";
        case DOBB_ERR_HIP: return "HIP launch failed";
        case DOBB_ERR_NOT_CONVERGED: return "eigensolver did not converge";
    }
    return "unknown status";
}

size_t dobb_workspace_size(dobb_op op, int count, const dobb_shape *shapes, int64_t N, int32_t variant) {
    if (count < 1 || !shapes) return 0;
    if (op != DOBB_OP_ACCUMULATE && op != DOBB_OP_REFRESH && op != DOBB_OP_STEP && op != DOBB_OP_STEP_G) return 0;
    if (op == DOBB_OP_ACCUMULATE && N < 1) return 0;
    if ((op == DOBB_OP_STEP || op == DOBB_OP_STEP_G) &&
        ((variant & ~DOBB_WS_BF16_BASIS) < 0 || (variant & ~DOBB_WS_BF16_BASIS) > 2))
        return 0;
    if (op == DOBB_OP_ACCUMULATE) variant = 0;
    if (op == DOBB_OP_REFRESH) variant &= DOBB_WS_BF16_BASIS;
    for (int i = 0; i < count; ++i)
        if ((op == DOBB_OP_STEP_G ? check_shape_g(&shapes[i]) : check_shape(&shapes[i])) != DOBB_OK) return 0;
    size_t need = 0;
    for (const auto &g : group_by_shape(count, shapes)) {
        size_t w = group_ws(op, shapes[g[0]], (int)g.size(), N, variant);
        if (w > need) need = w;
    }
    return need;
}

dobb_status dobb_accumulate_moment_grouped(int count, const dobb_shape *shapes, const void *const *X, dobb_dtype x_dtype,
                                           int64_t N, const int64_t *ldx, float beta, float *const *A, void *ws,
                                           size_t ws_bytes, dobb_stream_t stream) {
    if (count < 1 || !shapes || !X || !A) return DOBB_ERR_INVALID_ARG;
    if (x_dtype != DOBB_F32 && x_dtype != DOBB_BF16) return DOBB_ERR_DTYPE;
    if (N < 1 || !(beta >= 0.f && beta < 1.f)) return DOBB_ERR_INVALID_ARG;
    for (int i = 0; i < count; ++i) {
        dobb_status st = check_shape(&shapes[i]);
        if (st != DOBB_OK) return st;
        if (!X[i] || !A[i]) return DOBB_ERR_INVALID_ARG;
        if (ldx && ldx[i] < shapes[i].n) return DOBB_ERR_SHAPE;
    }
    const auto groups = group_by_shape(count, shapes);
    size_t need = 0;
    for (const auto &g : groups) { size_t w = group_ws(DOBB_OP_ACCUMULATE, shapes[g[0]], (int)g.size(), N, 0); if (w > need) need = w; }
    dobb_status st = check_ws(ws, ws_bytes, need);
    if (st != DOBB_OK) return st;
    for (const auto &g : groups) {
        std::vector<const void *> xs;
        std::vector<float *> as;
        std::vector<int64_t> lds;
        for (int i : g) { xs.push_back(X[i]); as.push_back(A[i]); lds.push_back(ldx ? ldx[i] : shapes[i].n); }
        AccumulateArgs a{};
        a.count = (int)g.size();
        a.sh = shapes[g[0]];
        a.x_dtype = x_dtype;
        a.N = N;
        a.ldx = lds.data();
        a.X = xs.data();
        a.A = as.data();
        a.beta = beta;
        a.nsplit = accumulate_splits(a.sh, N, a.count, x_dtype == DOBB_BF16);
        a.partial = (double *)ws;
        st = hip_status(launch_accumulate(a, (hipStream_t)stream));
        if (st != DOBB_OK) return st;
    }
    return DOBB_OK;
}

dobb_status dobb_accumulate_moment(const dobb_shape *s, const void *X, dobb_dtype x_dtype, int64_t N, int64_t ldx,
                                   float beta, float *A, void *ws, size_t ws_bytes, dobb_stream_t stream) {
    if (!s) return DOBB_ERR_INVALID_ARG;
    return dobb_accumulate_moment_grouped(1, s, &X, x_dtype, N, &ldx, beta, &A, ws, ws_bytes, stream);
}

dobb_status dobb_refresh_basis_grouped(int count, const dobb_shape *shapes, const float *const *A, void *const *Q,
                                       dobb_dtype q_dtype, float *const *lambda, dobb_refresh_mode mode, int iters,
                                       int warm_start, float tol, int32_t *const *info, void *ws, size_t ws_bytes,
                                       dobb_stream_t stream) {
    if (count < 1 || !shapes || !A || !Q) return DOBB_ERR_INVALID_ARG;
    if (q_dtype != DOBB_F32 && q_dtype != DOBB_BF16) return DOBB_ERR_DTYPE;
    if (mode != DOBB_REFRESH_EXACT && mode != DOBB_REFRESH_ORTH_ITER && mode != DOBB_REFRESH_ORTH_ITER_CHOLQR)
        return DOBB_ERR_INVALID_ARG;
    if (mode != DOBB_REFRESH_EXACT && iters < 1) return DOBB_ERR_INVALID_ARG;
    if (iters < 0 || iters > 1000) return DOBB_ERR_INVALID_ARG;
    if (!(tol >= 0.f) || tol >= 1.f) return DOBB_ERR_INVALID_ARG;
    for (int i = 0; i < count; ++i) {
        dobb_status st = check_shape(&shapes[i]);
        if (st != DOBB_OK) return st;
        if (!A[i] || !Q[i]) return DOBB_ERR_INVALID_ARG;
        if (mode == DOBB_REFRESH_ORTH_ITER_CHOLQR && !chol_supported(shapes[i].nb)) return DOBB_ERR_SHAPE;
    }
    const bool qbf = q_dtype == DOBB_BF16;
    const int variant = qbf ? DOBB_WS_BF16_BASIS : 0;
    const auto groups = group_by_shape(count, shapes);
    size_t need = 0;
    for (const auto &g : groups) { size_t w = group_ws(DOBB_OP_REFRESH, shapes[g[0]], (int)g.size(), 0, variant); if (w > need) need = w; }
    dobb_status st = check_ws(ws, ws_bytes, need);
    if (st != DOBB_OK) return st;
    hipStream_t hs = (hipStream_t)stream;
    for (const auto &g : groups) {
        const dobb_shape sh = shapes[g[0]];
        const int64_t elems = sh.n * sh.nb;
        for (size_t c0 = 0; c0 < g.size(); c0 += kMaxMats) {
            const int cnt = (int)(g.size() - c0 < (size_t)kMaxMats ? g.size() - c0 : (size_t)kMaxMats);
            // a bf16 basis is refreshed in an fp32 copy placed after the refresh regions
            char *copies = (char *)ws + al256(refresh_ws(sh, cnt));
            std::vector<const float *> as;
            std::vector<float *> qs, ls;
            std::vector<int32_t *> is;
            std::vector<const void *> qsrc;
            std::vector<void *> qdst;
            for (int k = 0; k < cnt; ++k) {
                const int i = g[c0 + k];
                as.push_back(A[i]);
                float *qf = qbf ? (float *)(copies + basis_copy_one(sh) * k) : (float *)Q[i];
                qs.push_back(qf);
                qsrc.push_back(Q[i]);
                qdst.push_back(qf);
                ls.push_back(lambda ? lambda[i] : nullptr);
                is.push_back(info ? info[i] : nullptr);
            }
            // warm starts and orthogonal iteration read the basis; a cold exact refresh does not
            if (qbf && (mode != DOBB_REFRESH_EXACT || warm_start)) {
                st = hip_status(launch_basis_convert(cnt, qsrc.data(), qdst.data(), elems, true, hs));
                if (st != DOBB_OK) return st;
            }
            RefreshArgs a{};
            a.count = cnt;
            a.sh = sh;
            a.A = as.data();
            a.Q = qs.data();
            a.lambda = ls.data();
            a.info = is.data();
            a.mode = mode;
            a.iters = mode == DOBB_REFRESH_EXACT ? (iters > 0 ? iters : 30) : iters;
            a.warm = warm_start ? 1 : 0;
            a.tol = tol > 0.f ? tol : 1e-7f;
            a.ws = ws;
            st = hip_status(launch_refresh(a, hs));
            if (st != DOBB_OK) return st;
            if (qbf) {
                std::vector<const void *> fsrc(qs.begin(), qs.end());
                std::vector<void *> bdst;
                for (int k = 0; k < cnt; ++k) bdst.push_back(Q[g[c0 + k]]);
                st = hip_status(launch_basis_convert(cnt, fsrc.data(), bdst.data(), elems, false, hs));
                if (st != DOBB_OK) return st;
            }
        }
    }
    return DOBB_OK;
}

dobb_status dobb_refresh_basis(const dobb_shape *s, const float *A, void *Q, dobb_dtype q_dtype, float *lambda,
                               dobb_refresh_mode mode, int iters, int warm_start, float tol, int32_t *info, void *ws,
                               size_t ws_bytes, dobb_stream_t stream) {
    if (!s) return DOBB_ERR_INVALID_ARG;
    return dobb_refresh_basis_grouped(1, s, &A, &Q, q_dtype, &lambda, mode, iters, warm_start, tol, &info, ws, ws_bytes,
                                      stream);
}

dobb_status dobb_step_grouped(int count, const dobb_shape *shapes, void *const *W, dobb_dtype w_dtype, const void *const *G,
                              dobb_dtype g_dtype, float *const *M, const void *const *Q, dobb_dtype q_dtype,
                              const dobb_hparams *hp, float *const *U_out, float *const *C_out, void *ws, size_t ws_bytes,
                              dobb_stream_t stream) {
    if (count < 1 || !shapes || !W || !G || !M || !Q || !hp) return DOBB_ERR_INVALID_ARG;
    if ((w_dtype != DOBB_F32 && w_dtype != DOBB_BF16) || (g_dtype != DOBB_F32 && g_dtype != DOBB_BF16) ||
        (q_dtype != DOBB_F32 && q_dtype != DOBB_BF16))
        return DOBB_ERR_DTYPE;
    for (int i = 0; i < count; ++i) {
        dobb_status st = check_shape(&shapes[i]);
        if (st != DOBB_OK) return st;
        if (!W[i] || !G[i] || !M[i] || !Q[i]) return DOBB_ERR_INVALID_ARG;
        if (hp[i].norm < 0 || hp[i].norm > 2) return DOBB_ERR_INVALID_ARG;
        if (hp[i].norm != hp[0].norm || (hp[i].nesterov != 0) != (hp[0].nesterov != 0)) return DOBB_ERR_INVALID_ARG;
    }
    const int norm = hp[0].norm;
    const bool qbf = q_dtype == DOBB_BF16;
    const int variant = norm | (qbf ? DOBB_WS_BF16_BASIS : 0);
    const auto groups = group_by_shape(count, shapes);
    size_t need = 0;
    for (const auto &g : groups) { size_t w = group_ws(DOBB_OP_STEP, shapes[g[0]], (int)g.size(), 0, variant); if (w > need) need = w; }
    dobb_status st = check_ws(ws, ws_bytes, need);
    if (st != DOBB_OK) return st;
    hipStream_t hs = (hipStream_t)stream;
    for (const auto &g : groups) {
        const dobb_shape sh = shapes[g[0]];
        const size_t per = step_region_one(sh, variant);
        const size_t own = step_ws_one(sh, norm);       // the step's regions; a basis copy follows them
        const bool bf16 = step_bf16_eligible(sh, norm);
        for (size_t c0 = 0; c0 < g.size(); c0 += kMaxMats) {
            const int cnt = (int)(g.size() - c0 < (size_t)kMaxMats ? g.size() - c0 : (size_t)kMaxMats);
            std::vector<const void *> gs, qsrc;
            std::vector<float *> ms, us, co, cs, ps;
            std::vector<double *> cps;
            std::vector<void *> ws_, qdst;
            std::vector<const float *> qs;
            std::vector<int8_t *> ss;
            std::vector<uint16_t *> pls;
            std::vector<dobb_hparams> hs_;
            bool aligned = true;
            for (int k = 0; k < cnt; ++k) {
                const int i = g[c0 + k];
                char *reg = (char *)ws + per * k;
                gs.push_back(G[i]); ms.push_back(M[i]); ws_.push_back(W[i]);
                us.push_back(U_out ? U_out[i] : nullptr);
                co.push_back(C_out ? C_out[i] : nullptr);
                hs_.push_back(hp[i]);
                float *qf = qbf ? (float *)(reg + own) : (float *)Q[i];
                qs.push_back(qf);
                qsrc.push_back(Q[i]);
                qdst.push_back(qf);
                ss.push_back((int8_t *)reg);
                cs.push_back((float *)reg);
                ps.push_back(norm == DOBB_NORM_SIGN ? nullptr : (float *)(reg + al256((size_t)sh.m * sh.n * 4)));
                cps.push_back(norm == DOBB_NORM_COL_L2
                                  ? (double *)(reg + al256((size_t)sh.m * sh.n * 4) + al256((size_t)sh.n * 4))
                                  : nullptr);
                const size_t s_bytes = al256((size_t)sh.m * (sh.n / sh.nb) * step_bf16_ldp(sh.nb));
                const size_t l2_planes = al256((size_t)sh.m * sh.n * 4) + al256((size_t)sh.n * 4) +
                                         al256((size_t)((sh.m + 127) / 128) * (size_t)sh.n * 8);
                pls.push_back(bf16 ? (uint16_t *)(reg + s_bytes)
                              : norm == DOBB_NORM_COL_L2 && step_wide_eligible(sh) ? (uint16_t *)(reg + l2_planes)
                                                                                    : nullptr);
                aligned = aligned && ((uintptr_t)M[i] & 15u) == 0 &&
                          ((uintptr_t)G[i] & (g_dtype == DOBB_BF16 ? 7u : 15u)) == 0 &&
                          ((uintptr_t)W[i] & (w_dtype == DOBB_BF16 ? 7u : 15u)) == 0 &&
                          ((uintptr_t)us.back() & 15u) == 0 && ((uintptr_t)co.back() & 15u) == 0;
            }
            if (qbf) {
                st = hip_status(launch_basis_convert(cnt, qsrc.data(), qdst.data(), sh.n * sh.nb, true, hs));
                if (st != DOBB_OK) return st;
            }
            StepArgs a{};
            a.count = cnt;
            a.sh = sh;
            a.w_dtype = w_dtype;
            a.g_dtype = g_dtype;
            a.hp = hs_.data();
            a.G = gs.data();
            a.M = ms.data();
            a.W = ws_.data();
            a.U = us.data();
            a.Cout = co.data();
            a.Q = qs.data();
            a.S = ss.data();
            a.C = cs.data();
            a.colscale = ps.data();
            a.colpart = cps.data();
            a.planes = pls.data();
            st = hip_status(bf16 && aligned ? launch_step_bf16(a, hs) : launch_step(a, hs));
            if (st != DOBB_OK) return st;
        }
    }
    return DOBB_OK;
}

dobb_status dobb_step(const dobb_shape *s, void *W, dobb_dtype w_dtype, const void *G, dobb_dtype g_dtype, float *M,
                      const void *Q, dobb_dtype q_dtype, const dobb_hparams *hp, float *U_out, float *C_out, void *ws,
                      size_t ws_bytes, dobb_stream_t stream) {
    if (!s) return DOBB_ERR_INVALID_ARG;
    return dobb_step_grouped(1, s, &W, w_dtype, &G, g_dtype, &M, &Q, q_dtype, hp, &U_out, &C_out, ws, ws_bytes, stream);
}

dobb_status dobb_step_g_grouped(int count, const dobb_shape *shapes, void *const *W, dobb_dtype w_dtype,
                                const void *const *G, dobb_dtype g_dtype, float *const *M, const void *const *P,
                                dobb_dtype p_dtype, const dobb_hparams *hp, float *const *U_out, float *const *C_out,
                                void *ws, size_t ws_bytes, dobb_stream_t stream) {
    if (count < 1 || !shapes || !W || !G || !M || !P || !hp) return DOBB_ERR_INVALID_ARG;
    if ((w_dtype != DOBB_F32 && w_dtype != DOBB_BF16) || (g_dtype != DOBB_F32 && g_dtype != DOBB_BF16) ||
        (p_dtype != DOBB_F32 && p_dtype != DOBB_BF16))
        return DOBB_ERR_DTYPE;
    for (int i = 0; i < count; ++i) {
        dobb_status st = check_shape_g(&shapes[i]);
        if (st != DOBB_OK) return st;
        if (!W[i] || !G[i] || !M[i] || !P[i]) return DOBB_ERR_INVALID_ARG;
        if (hp[i].norm < 0 || hp[i].norm > 2) return DOBB_ERR_INVALID_ARG;
        if (hp[i].norm != hp[0].norm || (hp[i].nesterov != 0) != (hp[0].nesterov != 0)) return DOBB_ERR_INVALID_ARG;
    }
    const int norm = hp[0].norm;
    const bool qbf = p_dtype == DOBB_BF16;
    const int variant = norm | (qbf ? DOBB_WS_BF16_BASIS : 0);
    const auto groups = group_by_shape(count, shapes);
    size_t need = 0;
    for (const auto &g : groups) { size_t w = group_ws(DOBB_OP_STEP_G, shapes[g[0]], (int)g.size(), 0, variant); if (w > need) need = w; }
    dobb_status st = check_ws(ws, ws_bytes, need);
    if (st != DOBB_OK) return st;
    hipStream_t hs = (hipStream_t)stream;
    for (const auto &g : groups) {
        const dobb_shape sh = shapes[g[0]];
        const size_t per = step_g_region_one(sh, variant);
        const size_t own = step_g_ws_one(sh, norm);
        const size_t mn4 = al256((size_t)sh.m * (size_t)sh.n * 4);
        const size_t chunk = (size_t)step_g_chunk(sh);
        for (size_t c0 = 0; c0 < g.size(); c0 += chunk) {
            const int cnt = (int)(g.size() - c0 < chunk ? g.size() - c0 : chunk);
            std::vector<const void *> gs, qsrc;
            std::vector<float *> ms, us, co, cs, rsc;
            std::vector<void *> ws_, qdst;
            std::vector<const float *> ps;
            std::vector<int8_t *> ss;
            std::vector<dobb_hparams> hs_;
            for (int k = 0; k < cnt; ++k) {
                const int i = g[c0 + k];
                char *reg = (char *)ws + per * k;
                gs.push_back(G[i]); ms.push_back(M[i]); ws_.push_back(W[i]);
                us.push_back(U_out ? U_out[i] : nullptr);
                co.push_back(C_out ? C_out[i] : nullptr);
                hs_.push_back(hp[i]);
                float *pf = qbf ? (float *)(reg + own) : (float *)P[i];
                ps.push_back(pf);
                qsrc.push_back(P[i]);
                qdst.push_back(pf);
                ss.push_back((int8_t *)reg);
                cs.push_back((float *)reg);
                rsc.push_back(norm == DOBB_NORM_SIGN ? nullptr : (float *)(reg + mn4));
            }
            if (qbf) {
                st = hip_status(launch_basis_convert(cnt, qsrc.data(), qdst.data(), sh.m * sh.nb, true, hs));
                if (st != DOBB_OK) return st;
            }
            StepArgs a{};
            a.count = cnt;
            a.sh = sh;
            a.w_dtype = w_dtype;
            a.g_dtype = g_dtype;
            a.hp = hs_.data();
            a.G = gs.data();
            a.M = ms.data();
            a.W = ws_.data();
            a.U = us.data();
            a.Cout = co.data();
            a.Q = ps.data();
            a.S = ss.data();
            a.C = cs.data();
            a.colscale = rsc.data();
            st = hip_status(launch_step_g(a, hs));
            if (st != DOBB_OK) return st;
        }
    }
    return DOBB_OK;
}

dobb_status dobb_step_g(const dobb_shape *s, void *W, dobb_dtype w_dtype, const void *G, dobb_dtype g_dtype, float *M,
                        const void *P, dobb_dtype p_dtype, const dobb_hparams *hp, float *U_out, float *C_out, void *ws,
                        size_t ws_bytes, dobb_stream_t stream) {
    if (!s) return DOBB_ERR_INVALID_ARG;
    return dobb_step_g_grouped(1, s, &W, w_dtype, &G, g_dtype, &M, &P, p_dtype, hp, &U_out, &C_out, ws, ws_bytes, stream);
}

dobb_status dobb_step_noalloc(const dobb_shape *s, void *W, dobb_dtype w_dtype, const void *G, dobb_dtype g_dtype,
                              float *M, const void *Q, dobb_dtype q_dtype, const dobb_hparams *hp, float *U_out,
                              float *C_out, dobb_stream_t stream) {
    // everything that can be refused is refused before the first HIP call
    if (!s || !hp || !W || !G || !M || !Q) return DOBB_ERR_INVALID_ARG;
    dobb_status st = check_shape(s);
    if (st != DOBB_OK) return st;
    if ((w_dtype != DOBB_F32 && w_dtype != DOBB_BF16) || (g_dtype != DOBB_F32 && g_dtype != DOBB_BF16) ||
        (q_dtype != DOBB_F32 && q_dtype != DOBB_BF16))
        return DOBB_ERR_DTYPE;
    if (hp->norm < 0 || hp->norm > 2) return DOBB_ERR_INVALID_ARG;
    const size_t need = group_ws(DOBB_OP_STEP, *s, 1, 0, hp->norm | (q_dtype == DOBB_BF16 ? DOBB_WS_BF16_BASIS : 0));
    if (need > (size_t)DOBB_NOALLOC_SCRATCH_BYTES) return DOBB_ERR_WORKSPACE;
    void *ws = nullptr;
    st = scratch_for_current_device(&ws);
    if (st != DOBB_OK) return st;
    return dobb_step_grouped(1, s, &W, w_dtype, &G, g_dtype, &M, &Q, q_dtype, hp, &U_out, &C_out, ws,
                             (size_t)DOBB_NOALLOC_SCRATCH_BYTES, stream);
}

void dobb_profile_enable(int on) {
    if (!on) prof_collect();
    prof().on = on != 0;
}

int dobb_profile_read(const char **names, int64_t *launches, double *total_ms, int cap) {
    prof_collect();
    const auto &t = prof().totals;
    const int n = (int)t.size();
    for (int i = 0; i < n && i < cap; ++i) {
        if (names) names[i] = std::get<0>(t[i]);
        if (launches) launches[i] = std::get<1>(t[i]);
        if (total_ms) total_ms[i] = std::get<2>(t[i]);
    }
    return n;
}

void dobb_profile_reset(void) {
    prof_collect();
    prof().totals.clear();
}

}  // extern "C"
