// api.hip -- the C ABI of libcsa.so (declared in include/csa.h): host-side
// argument checks, workspace sizing and kernel launches.  Nothing here
// allocates, frees or synchronises.
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "csa.h"
#include "common.h"
#include "internal.h"

namespace csa {
int64_t index_merge_max();
}

namespace {

thread_local char g_err[512] = "";

csa_status fail(csa_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return st;
}

csa_status ok() {
    g_err[0] = '\0';
    return CSA_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

csa_status launched(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(CSA_EDEVICE, "%s: launch failed: %s", what, hipGetErrorString(e));
    return ok();
}

#define CHECK(cond, st, ...) \
    do { if (!(cond)) return fail(st, __VA_ARGS__); } while (0)

csa_status check_dtype(csa_dtype dt, const char* fn) {
    CHECK(dt == CSA_F32 || dt == CSA_BF16, CSA_EINVAL, "%s: unknown dtype %d", fn, (int)dt);
    return CSA_OK;
}

// The window of every query must lie inside the raw rows, the compressed
// tensors must hold every candidate, and the key list must be non-empty.
csa_status check_positions(const char* fn, int64_t Tq, int64_t Nc, int64_t m, int64_t W,
                           int64_t q_pos0, int64_t raw_pos0, int64_t raw_len) {
    CHECK(m >= 1, CSA_EINVAL, "%s: m must be >= 1 (got %lld)", fn, (long long)m);
    CHECK(W >= 1, CSA_EINVAL, "%s: window W must be >= 1 (got %lld)", fn, (long long)W);
    CHECK(q_pos0 >= 0, CSA_EINVAL, "%s: q_pos0 must be >= 0", fn);
    CHECK(Nc >= 0 && Nc < ((int64_t)1 << 31), CSA_EINVAL, "%s: Nc out of range", fn);
    if (Tq == 0) return CSA_OK;
    const int64_t tlast = q_pos0 + Tq - 1;
    const int64_t need = csa::n_candidates(tlast, m, W);
    CHECK(need <= Nc, CSA_EINVAL, "%s: query at %lld has %lld candidates but Nc = %lld", fn,
          (long long)tlast, (long long)need, (long long)Nc);
    if (raw_len >= 0) {
        const int64_t w0 = q_pos0 - W + 1 < 0 ? 0 : q_pos0 - W + 1;
        CHECK(raw_pos0 >= 0 && w0 >= raw_pos0 && tlast < raw_pos0 + raw_len, CSA_EINVAL,
              "%s: raw rows [%lld, %lld) do not cover the windows [%lld, %lld]", fn,
              (long long)raw_pos0, (long long)(raw_pos0 + raw_len), (long long)w0,
              (long long)tlast);
    }
    return CSA_OK;
}

// A strided view as the kernels take it (element strides)
csa::RowStrides strides(const csa_in& v) { return {v.seq_stride, v.row_stride}; }
csa::RowStrides strides(const csa_out& v) { return {v.seq_stride, v.row_stride}; }

// A dense [B][rows][row_elems] tensor as a view
csa_in dense_in(const void* p, int64_t rows, int64_t row_elems) {
    return csa_in{p, rows * row_elems, row_elems};
}
csa_out dense_out(void* p, int64_t rows, int64_t row_elems) {
    return csa_out{p, rows * row_elems, row_elems};
}

// A view of B sequences of `rows` rows of `row_elems` contiguous elements of
// esize bytes: non-negative strides, rows that do not overlap, and (align)
// base and strides on 16-byte boundaries; an output's sequences must not
// overlap either.
csa_status check_view(const char* fn, const char* name, const void* p, int64_t ss, int64_t rs,
                      int64_t B, int64_t rows, int64_t row_elems, int64_t esize, bool out,
                      bool align = true) {
    CHECK(p, CSA_EINVAL, "%s: null pointer (%s)", fn, name);
    CHECK(ss >= 0 && rs >= 0, CSA_EINVAL, "%s: %s: strides must be >= 0", fn, name);
    CHECK(rows <= 1 || rs >= row_elems, CSA_EINVAL,
          "%s: %s: row stride %lld is below the row length %lld", fn, name, (long long)rs,
          (long long)row_elems);
    CHECK(!align || (((uintptr_t)p & 15u) == 0 && (ss * esize) % 16 == 0 && (rs * esize) % 16 == 0),
          CSA_EINVAL, "%s: %s: base and strides must be 16-byte aligned", fn, name);
    if (out && B > 1 && rows > 0)
        CHECK(ss >= (rows - 1) * rs + row_elems, CSA_EINVAL,
              "%s: %s: sequence stride %lld makes sequences overlap", fn, name, (long long)ss);
    return CSA_OK;
}

}  // namespace

extern "C" {

int csa_abi_version(void) { return CSA_ABI_VERSION; }

const char* csa_last_error(void) { return g_err; }

csa_status hca_compress(csa_dtype dt, int64_t B, int64_t T, int64_t C, int64_t m, csa_in x,
                        csa_in gate, int64_t gate_channels, csa_out out, hipStream_t stream) {
    const char* fn = "hca_compress";
    if (csa_status s = check_dtype(dt, fn)) return s;
    CHECK(B >= 1 && B < 65536 * 1024LL, CSA_EINVAL, "%s: B out of range", fn);
    CHECK(T >= 0, CSA_EINVAL, "%s: T must be >= 0", fn);
    CHECK(m >= 1, CSA_EINVAL, "%s: m must be >= 1", fn);
    CHECK(C >= 8 && C % 8 == 0 && C <= 1024, CSA_EINVAL,
          "%s: C must be a multiple of 8 in [8, 1024] (got %lld)", fn, (long long)C);
    CHECK(gate_channels == 1 || gate_channels == C, CSA_EINVAL,
          "%s: gate_channels must be 1 or C", fn);
    const int64_t esz = dt == CSA_F32 ? 4 : 2;
    if (csa_status s = check_view(fn, "x", x.p, x.seq_stride, x.row_stride, B, T, C, esz, false))
        return s;
    if (csa_status s = check_view(fn, "gate", gate.p, gate.seq_stride, gate.row_stride, B, T,
                                  gate_channels, esz, false, gate_channels != 1))
        return s;
    if (csa_status s = check_view(fn, "out", out.p, out.seq_stride, out.row_stride, B, T / m, C,
                                  esz, true))
        return s;
    const int64_t blocks = (m <= 16) ? (B * (T / m) * (C / 8) + 255) / 256 : B * (T / m);
    CHECK(blocks < ((int64_t)1 << 31), CSA_EUNSUPPORTED, "%s: problem too large", fn);
    return launched(csa::launch_compress((int)dt, x.p, strides(x), gate.p, strides(gate), out.p,
                                         strides(out), B, T, (int)C, (int)m, (int)gate_channels,
                                         stream),
                    fn);
}

csa_status hca_append(csa_dtype dt, int64_t B, int64_t C, int64_t m, int64_t W, int64_t t,
                      const void* k_new, const void* v_new, const void* gk_new,
                      const void* gv_new, int64_t gate_channels, void* rk, void* rv,
                      int64_t wcap, int64_t* win_pos0, void* gk_blk, void* gv_blk, void* ck,
                      void* cv, int64_t nc_cap, hipStream_t stream) {
    const char* fn = "hca_append";
    if (csa_status s = check_dtype(dt, fn)) return s;
    CHECK(win_pos0, CSA_EINVAL, "%s: null pointer", fn);
    CHECK(B >= 1 && B < 65536 * 1024LL, CSA_EINVAL, "%s: B out of range", fn);
    CHECK(C >= 8 && C % 8 == 0 && C <= 1024, CSA_EINVAL,
          "%s: C must be a multiple of 8 in [8, 1024] (got %lld)", fn, (long long)C);
    CHECK(m >= 1 && W >= m, CSA_EINVAL, "%s: need 1 <= m <= W (got m = %lld, W = %lld)", fn,
          (long long)m, (long long)W);
    CHECK(wcap >= 2 * W && wcap < ((int64_t)1 << 31) / C, CSA_EINVAL,
          "%s: the window buffer needs 2W <= wcap rows (got %lld)", fn, (long long)wcap);
    CHECK(gate_channels == 1 || gate_channels == C, CSA_EINVAL,
          "%s: gate_channels must be 1 or C", fn);
    const int64_t p0 = *win_pos0;
    const int64_t keep = t < W - 1 ? t : W - 1;          // rows the window buffer must hold
    CHECK(t >= 0 && p0 >= 0 && p0 <= t - keep && t - p0 <= wcap, CSA_EINVAL,
          "%s: the window buffer holds positions %lld .. %lld but token %lld needs its %lld "
          "predecessors and at most %lld rows",
          fn, (long long)p0, (long long)t - 1, (long long)t, (long long)keep, (long long)wcap);
    CHECK(nc_cap >= (t + 1) / m && nc_cap < ((int64_t)1 << 31) / C, CSA_EINVAL,
          "%s: nc_cap = %lld cannot hold entry %lld", fn, (long long)nc_cap,
          (long long)((t + 1) / m - 1));
    CHECK(k_new && v_new && gk_new && gv_new && rk && rv && gk_blk && gv_blk && ck && cv,
          CSA_EINVAL, "%s: null pointer", fn);
    CHECK(aligned16(k_new) && aligned16(v_new) && aligned16(rk) && aligned16(rv) &&
              aligned16(ck) && aligned16(cv) &&
              (gate_channels == 1 ||
               (aligned16(gk_new) && aligned16(gv_new) && aligned16(gk_blk) && aligned16(gv_blk))),
          CSA_EINVAL, "%s: rows (and per-channel gates) must be 16-byte aligned", fn);
    int64_t np0 = p0;
    const csa_status st = launched(
        csa::launch_append((int)dt, B, C, m, W, t, p0, wcap, gate_channels, nc_cap, k_new, v_new,
                           gk_new, gv_new, rk, rv, gk_blk, gv_blk, ck, cv, &np0, stream),
        fn);
    if (st == CSA_OK) *win_pos0 = np0;
    return st;
}

csa_status csa_quantize_mxfp4(csa_dtype dt, int64_t rows, int64_t d, csa_in x, uint8_t* codes,
                              uint8_t* scales, hipStream_t stream) {
    const char* fn = "csa_quantize_mxfp4";
    if (csa_status s = check_dtype(dt, fn)) return s;
    CHECK(rows >= 0, CSA_EINVAL, "%s: rows must be >= 0", fn);
    CHECK(d >= 32 && d % 32 == 0, CSA_EINVAL, "%s: d must be a positive multiple of 32", fn);
    const int64_t esz = dt == CSA_F32 ? 4 : 2;
    if (csa_status s = check_view(fn, "x", x.p, 0, x.row_stride, 1, rows, d, esz, false))
        return s;
    CHECK(codes && scales, CSA_EINVAL, "%s: null pointer", fn);
    CHECK(aligned16(codes), CSA_EINVAL, "%s: codes must be 16-byte aligned", fn);
    CHECK((rows * (d / 32) + 255) / 256 < ((int64_t)1 << 31), CSA_EUNSUPPORTED,
          "%s: problem too large", fn);
    return launched(csa::launch_quant_mxfp4((int)dt, x.p, x.row_stride, codes, scales, rows,
                                            (int)d, stream),
                    fn);
}

static csa_status index_args(const char* fn, int64_t B, int64_t Tq, int64_t HI, int64_t dI,
                             int64_t Nc, int64_t m, int64_t W, int64_t k, int64_t q_pos0) {
    CHECK(B >= 1 && B < 65536, CSA_EINVAL, "%s: B must be in [1, 65535]", fn);
    CHECK(Tq >= 0, CSA_EINVAL, "%s: Tq must be >= 0", fn);
    CHECK(HI == 1 || HI == 2 || HI == 4, CSA_EUNSUPPORTED, "%s: HI must be 1, 2 or 4", fn);
    CHECK(dI == 32 || dI == 64, CSA_EUNSUPPORTED, "%s: dI must be 32 or 64", fn);
    CHECK(k >= 1 && k <= 2048, CSA_EINVAL, "%s: k must be in [1, 2048]", fn);
    if (csa_status s = check_positions(fn, Tq, Nc, m, W, q_pos0, 0, -1)) return s;
    csa::IndexPlan p = csa::plan_index(B, Tq, (int)HI, (int)dI, Nc, m, W, (int)k, q_pos0);
    CHECK(p.n_qtiles < 65536, CSA_EUNSUPPORTED, "%s: too many query rows", fn);
    CHECK(p.n_chunks < ((int64_t)1 << 31), CSA_EUNSUPPORTED, "%s: too many candidates", fn);
    CHECK(p.path != csa::IDX_CHUNK || p.n_chunks == 1 || p.n_chunks * k <= csa::index_merge_max(),
          CSA_EUNSUPPORTED,
          "%s: %lld candidate chunks x k = %lld exceeds the merge limit %lld", fn,
          (long long)p.n_chunks, (long long)k, (long long)csa::index_merge_max());
    return CSA_OK;
}

csa_status csa_index_topk_workspace(int64_t B, int64_t Tq, int64_t HI, int64_t dI, int64_t Nc,
                                    int64_t m, int64_t W, int64_t k, int64_t q_pos0,
                                    size_t* bytes) {
    const char* fn = "csa_index_topk_workspace";
    CHECK(bytes, CSA_EINVAL, "%s: null pointer", fn);
    if (csa_status s = index_args(fn, B, Tq, HI, dI, Nc, m, W, k, q_pos0)) return s;
    *bytes = csa::plan_index(B, Tq, (int)HI, (int)dI, Nc, m, W, (int)k, q_pos0).ws_bytes;
    return ok();
}

// run == false: every check of the entry point, no launch
static csa_status index_topk_do(bool run, const char* fn, csa_dtype dt, int64_t B, int64_t Tq,
                                int64_t HI, int64_t dI, int64_t Nc, int64_t m, int64_t W,
                                int64_t k, int64_t q_pos0, csa_in q_idx,
                                const uint8_t* k_codes, const uint8_t* k_scales, int32_t* topk,
                                void* ws, size_t ws_bytes, hipStream_t stream) {
    if (csa_status s = check_dtype(dt, fn)) return s;
    if (csa_status s = index_args(fn, B, Tq, HI, dI, Nc, m, W, k, q_pos0)) return s;
    const int64_t esz = dt == CSA_F32 ? 4 : 2;
    if (csa_status s = check_view(fn, "q_idx", q_idx.p, q_idx.seq_stride, q_idx.row_stride, B,
                                  Tq, HI * dI, esz, false))
        return s;
    CHECK(k_codes && k_scales && topk, CSA_EINVAL, "%s: null pointer", fn);
    CHECK(aligned16(k_codes), CSA_EINVAL, "%s: k_codes must be 16-byte aligned", fn);
    csa::IndexPlan p = csa::plan_index(B, Tq, (int)HI, (int)dI, Nc, m, W, (int)k, q_pos0);
    CHECK(ws_bytes >= p.ws_bytes && (p.ws_bytes == 0 || (ws && aligned16(ws))), CSA_EINVAL,
          "%s: workspace of %zu bytes given, %zu needed", fn, ws_bytes, p.ws_bytes);
    if (!run) return CSA_OK;
    return launched(csa::launch_index_topk((int)dt, p, B, Tq, (int)HI, (int)dI, Nc, m, W, (int)k,
                                           q_pos0, q_idx.p, strides(q_idx), k_codes, k_scales,
                                           topk, ws, stream),
                    fn);
}

csa_status csa_index_topk(csa_dtype dt, int64_t B, int64_t Tq, int64_t HI, int64_t dI,
                          int64_t Nc, int64_t m, int64_t W, int64_t k, int64_t q_pos0,
                          csa_in q_idx, const uint8_t* k_codes, const uint8_t* k_scales,
                          int32_t* topk, void* ws, size_t ws_bytes, hipStream_t stream) {
    return index_topk_do(true, "csa_index_topk", dt, B, Tq, HI, dI, Nc, m, W, k, q_pos0, q_idx,
                         k_codes, k_scales, topk, ws, ws_bytes, stream);
}

// ---- selection without a workspace argument ---------------------------------
// The static scratch array of csa_index_topk_noalloc.  In host code its name
// is only a stand-in: kernels receive the per-device address that
// hipGetSymbolAddress returns for it.
static __device__ __align__(256) unsigned char scratch[CSA_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_DEVICES];          // per device, looked up once
}  // namespace

static csa_status scratch_ptr(const char* fn, void** p) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return fail(CSA_EDEVICE, "%s: no current device", fn);
    CHECK(dev >= 0 && dev < MAX_DEVICES, CSA_EUNSUPPORTED, "%s: device %d out of range", fn, dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* q = nullptr;
        const hipError_t e = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !q)
            return fail(CSA_EDEVICE, "%s: scratch address lookup failed: %s", fn,
                        hipGetErrorString(e));
        g_scratch_ptr[dev] = q;
    }
    *p = g_scratch_ptr[dev];
    return CSA_OK;
}

csa_status csa_index_topk_noalloc(csa_dtype dt, int64_t B, int64_t Tq, int64_t HI, int64_t dI,
                                  int64_t Nc, int64_t m, int64_t W, int64_t k, int64_t q_pos0,
                                  csa_in q_idx, const uint8_t* k_codes,
                                  const uint8_t* k_scales, int32_t* topk,
                                  hipStream_t stream) {
    const char* fn = "csa_index_topk_noalloc";
    // every check of csa_index_topk first (no device call), then the size
    void* fake_ws = (void*)(uintptr_t)256;
    if (csa_status s = index_topk_do(false, fn, dt, B, Tq, HI, dI, Nc, m, W, k, q_pos0, q_idx,
                                     k_codes, k_scales, topk, fake_ws, SIZE_MAX, stream))
        return s;
    const size_t need =
        csa::plan_index(B, Tq, (int)HI, (int)dI, Nc, m, W, (int)k, q_pos0).ws_bytes;
    CHECK(need <= CSA_NOALLOC_SCRATCH_BYTES, CSA_EUNSUPPORTED,
          "%s: the selection needs %zu bytes of scratch, the static array holds %zu "
          "(use csa_index_topk with a workspace)",
          fn, need, (size_t)CSA_NOALLOC_SCRATCH_BYTES);
    void* ws = nullptr;
    if (need > 0)
        if (csa_status s = scratch_ptr(fn, &ws)) return s;
    return index_topk_do(true, fn, dt, B, Tq, HI, dI, Nc, m, W, k, q_pos0, q_idx, k_codes,
                         k_scales, topk, ws, need, stream);
}

static csa_status attend_shape(const char* fn, csa_dtype dt, int64_t B, int64_t Tq, int64_t H,
                               int64_t D) {
    if (csa_status s = check_dtype(dt, fn)) return s;
    CHECK(B >= 1 && B < 65536, CSA_EINVAL, "%s: B must be in [1, 65535]", fn);
    CHECK(Tq >= 0 && Tq < ((int64_t)1 << 31), CSA_EINVAL, "%s: Tq out of range", fn);
    CHECK(H >= 1 && D >= 1, CSA_EINVAL, "%s: H and D must be >= 1", fn);
    if (dt == CSA_BF16) {
        CHECK(H % 32 == 0 && (H / 32 == 1 || H / 32 == 2 || H / 32 == 4 || H / 32 == 8),
              CSA_EUNSUPPORTED, "%s: bf16 needs H in {32, 64, 128, 256} (got %lld)", fn,
              (long long)H);
        CHECK(D == 64 || D == 128, CSA_EUNSUPPORTED, "%s: bf16 needs D in {64, 128}", fn);
    } else {
        CHECK(D <= 256, CSA_EUNSUPPORTED, "%s: fp32 needs D <= 256", fn);
    }
    return CSA_OK;
}

// The bf16 attention kernel addresses key and value rows with 32-bit byte
// offsets from their sequence's base and key-list positions with 32-bit ints.
static csa_status attend_ranges(const char* fn, int64_t Nc, int64_t D, int64_t raw_len, int64_t k,
                                int64_t W, int64_t q_pos0, int64_t Tq, int64_t m) {
    const int64_t lim = ((int64_t)1 << 31) - 1;
    CHECK(Nc * D * 2 <= lim && raw_len * D * 2 <= lim, CSA_EUNSUPPORTED,
          "%s: caches larger than 2 GiB per sequence are not supported", fn);
    const int64_t keys = (Tq > 0 ? csa::n_candidates(q_pos0 + Tq - 1, m, W) : 0) + k + W;
    CHECK(keys <= lim, CSA_EUNSUPPORTED, "%s: key list too long", fn);
    return CSA_OK;
}

// The views of one attention call: q / o rows are query tokens of [H][D]
// contiguous elements, ck / cv rows compressed entries and rk / rv rows raw
// tokens of D contiguous elements; a sequence's key and value rows must lie
// within 2 GiB of its first row.
static csa_status attend_views(const char* fn, csa_dtype dt, int64_t B, int64_t Tq, int64_t H,
                               int64_t D, int64_t Nc, int64_t raw_len, const csa_in& q,
                               const csa_in& ck, const csa_in& cv, const csa_in& rk,
                               const csa_in& rv, const csa_out& o) {
    const int64_t esz = dt == CSA_F32 ? 4 : 2;
    if (csa_status s = check_view(fn, "q", q.p, q.seq_stride, q.row_stride, B, Tq, H * D, esz,
                                  false))
        return s;
    const csa_in* kv[4] = {&ck, &cv, &rk, &rv};
    const char* names[4] = {"ck", "cv", "rk", "rv"};
    for (int i = 0; i < 4; ++i) {
        const int64_t rows = i < 2 ? Nc : raw_len;
        if (csa_status s = check_view(fn, names[i], kv[i]->p, kv[i]->seq_stride,
                                      kv[i]->row_stride, B, rows, D, esz, false))
            return s;
        CHECK(rows == 0 || (rows - 1) * kv[i]->row_stride * esz + D * esz <= ((int64_t)1 << 31) - 1,
              CSA_EUNSUPPORTED, "%s: %s: a sequence's rows span more than 2 GiB", fn, names[i]);
    }
    return check_view(fn, "o", o.p, o.seq_stride, o.row_stride, B, Tq, H * D, esz, true);
}

static csa::AttendIO attend_io(const csa_in& q, const csa_in& ck, const csa_in& cv,
                               const csa_in& rk, const csa_in& rv, const csa_out& o) {
    return csa::AttendIO{q.p,          ck.p,          cv.p,          rk.p,        rv.p,
                         o.p,          strides(q),    strides(ck),   strides(cv), strides(rk),
                         strides(rv),  strides(o)};
}

csa_status csa_attend_workspace(csa_dtype dt, int64_t B, int64_t Tq, int64_t H, int64_t D,
                                int64_t k, int64_t W, size_t* bytes) {
    const char* fn = "csa_attend_workspace";
    CHECK(bytes, CSA_EINVAL, "%s: null pointer", fn);
    if (csa_status s = attend_shape(fn, dt, B, Tq, H, D)) return s;
    CHECK(k >= 1 && k <= 2048 && W >= 1, CSA_EINVAL, "%s: need 1 <= k <= 2048 and W >= 1", fn);
    *bytes = csa::plan_attend((int)dt, B, Tq, H, D, k + W).ws_bytes;
    return ok();
}

static csa_status csa_attend_do(bool run, const char* fn, csa_dtype dt, int64_t B, int64_t Tq,
                                int64_t H, int64_t D, int64_t Nc, int64_t m, int64_t W,
                                int64_t k, int64_t q_pos0, float scale, csa_in q, csa_in ck,
                                csa_in cv, const int32_t* topk, csa_in rk, csa_in rv,
                                int64_t raw_pos0, int64_t raw_len, csa_out o, void* ws,
                                size_t ws_bytes, hipStream_t stream) {
    if (csa_status s = attend_shape(fn, dt, B, Tq, H, D)) return s;
    CHECK(k >= 1 && k <= 2048, CSA_EINVAL, "%s: k must be in [1, 2048]", fn);
    CHECK(raw_len >= 0, CSA_EINVAL, "%s: raw_len must be >= 0", fn);
    CHECK(topk, CSA_EINVAL, "%s: null pointer", fn);
    if (csa_status s = attend_views(fn, dt, B, Tq, H, D, Nc, raw_len, q, ck, cv, rk, rv, o))
        return s;
    if (csa_status s = check_positions(fn, Tq, Nc, m, W, q_pos0, raw_pos0, raw_len)) return s;
    if (csa_status s = attend_ranges(fn, Nc, D, raw_len, k, W, q_pos0, Tq, m)) return s;
    csa::AttendPlan p = csa::plan_attend((int)dt, B, Tq, H, D, k + W);
    CHECK(ws_bytes >= p.ws_bytes && (p.ws_bytes == 0 || (ws && aligned16(ws))), CSA_EINVAL,
          "%s: workspace of %zu bytes given, %zu needed", fn, ws_bytes, p.ws_bytes);
    if (!run) return CSA_OK;
    return launched(csa::launch_attend((int)dt, p, B, Tq, H, D, Nc, m, W, k, q_pos0, scale,
                                       attend_io(q, ck, cv, rk, rv, o), topk, raw_pos0, raw_len,
                                       ws, stream),
                    fn);
}

csa_status csa_attend(csa_dtype dt, int64_t B, int64_t Tq, int64_t H, int64_t D, int64_t Nc,
                      int64_t m, int64_t W, int64_t k, int64_t q_pos0, float scale, csa_in q,
                      csa_in ck, csa_in cv, const int32_t* topk, csa_in rk, csa_in rv,
                      int64_t raw_pos0, int64_t raw_len, csa_out o, void* ws, size_t ws_bytes,
                      hipStream_t stream) {
    return csa_attend_do(true, "csa_attend", dt, B, Tq, H, D, Nc, m, W, k, q_pos0, scale, q, ck,
                         cv, topk, rk, rv, raw_pos0, raw_len, o, ws, ws_bytes, stream);
}

static int64_t hca_max_keys(int64_t Tq, int64_t m, int64_t W, int64_t q_pos0) {
    return (Tq > 0 ? csa::n_candidates(q_pos0 + Tq - 1, m, W) : 0) + W;
}

csa_status hca_attend_workspace(csa_dtype dt, int64_t B, int64_t Tq, int64_t H, int64_t D,
                                int64_t Nc, int64_t m, int64_t W, int64_t q_pos0,
                                size_t* bytes) {
    const char* fn = "hca_attend_workspace";
    CHECK(bytes, CSA_EINVAL, "%s: null pointer", fn);
    if (csa_status s = attend_shape(fn, dt, B, Tq, H, D)) return s;
    if (csa_status s = check_positions(fn, Tq, Nc, m, W, q_pos0, 0, -1)) return s;
    *bytes = csa::plan_attend((int)dt, B, Tq, H, D, hca_max_keys(Tq, m, W, q_pos0)).ws_bytes;
    return ok();
}

static csa_status hca_attend_do(bool run, const char* fn, csa_dtype dt, int64_t B, int64_t Tq,
                                int64_t H, int64_t D, int64_t Nc, int64_t m, int64_t W,
                                int64_t q_pos0, float scale, csa_in q, csa_in ck, csa_in cv,
                                csa_in rk, csa_in rv, int64_t raw_pos0, int64_t raw_len,
                                csa_out o, void* ws, size_t ws_bytes, hipStream_t stream) {
    if (csa_status s = attend_shape(fn, dt, B, Tq, H, D)) return s;
    CHECK(raw_len >= 0, CSA_EINVAL, "%s: raw_len must be >= 0", fn);
    if (csa_status s = attend_views(fn, dt, B, Tq, H, D, Nc, raw_len, q, ck, cv, rk, rv, o))
        return s;
    if (csa_status s = check_positions(fn, Tq, Nc, m, W, q_pos0, raw_pos0, raw_len)) return s;
    if (csa_status s = attend_ranges(fn, Nc, D, raw_len, 0, W, q_pos0, Tq, m)) return s;
    csa::AttendPlan p = csa::plan_attend((int)dt, B, Tq, H, D, hca_max_keys(Tq, m, W, q_pos0));
    CHECK(ws_bytes >= p.ws_bytes && (p.ws_bytes == 0 || (ws && aligned16(ws))), CSA_EINVAL,
          "%s: workspace of %zu bytes given, %zu needed", fn, ws_bytes, p.ws_bytes);
    if (!run) return CSA_OK;
    return launched(csa::launch_attend((int)dt, p, B, Tq, H, D, Nc, m, W, 0, q_pos0, scale,
                                       attend_io(q, ck, cv, rk, rv, o), nullptr, raw_pos0,
                                       raw_len, ws, stream),
                    fn);
}

csa_status hca_attend(csa_dtype dt, int64_t B, int64_t Tq, int64_t H, int64_t D, int64_t Nc,
                      int64_t m, int64_t W, int64_t q_pos0, float scale, csa_in q, csa_in ck,
                      csa_in cv, csa_in rk, csa_in rv, int64_t raw_pos0, int64_t raw_len,
                      csa_out o, void* ws, size_t ws_bytes, hipStream_t stream) {
    return hca_attend_do(true, "hca_attend", dt, B, Tq, H, D, Nc, m, W, q_pos0, scale, q, ck, cv,
                         rk, rv, raw_pos0, raw_len, o, ws, ws_bytes, stream);
}

// ---- one CSA layer's selection and attention, pipelined over query slices ----

static size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

struct SliceWs {
    size_t index, attend;   // bytes of the two regions (index first)
};

// The attention of every slice keeps the key-list splits of the whole call,
// so each row is computed exactly as csa_attend computes it.
static csa::AttendPlan slice_attend_plan(csa_dtype dt, int64_t B, int64_t Tq, int64_t rows,
                                         int64_t H, int64_t D, int64_t k, int64_t W) {
    csa::AttendPlan p = csa::plan_attend((int)dt, B, Tq, H, D, k + W);
    p.ws_bytes = p.splits > 1 ? (size_t)(rows * p.splits * H) * (D * 2 + 8) : 0;
    return p;
}

// query rows a .. b of one sequence form a slice; slices are ceil(Tq / n) rows
static SliceWs slice_ws(csa_dtype dt, int64_t B, int64_t Tq, int64_t H, int64_t D, int64_t HI,
                        int64_t dI, int64_t Nc, int64_t m, int64_t W, int64_t k, int64_t q_pos0,
                        int64_t n_chunks) {
    SliceWs r{0, 0};
    const int64_t per = (Tq + n_chunks - 1) / n_chunks;
    for (int64_t a = 0; a < Tq; a += per) {
        const int64_t rows = Tq - a < per ? Tq - a : per;
        const size_t i = csa::plan_index(1, rows, (int)HI, (int)dI, Nc, m, W, (int)k, q_pos0 + a)
                             .ws_bytes;
        const size_t t = slice_attend_plan(dt, B, Tq, rows, H, D, k, W).ws_bytes;
        r.index = i > r.index ? i : r.index;
        r.attend = t > r.attend ? t : r.attend;
    }
    return r;
}

// The events of one pipelined call: created at its start, destroyed when it
// returns (no event outlives the call).
struct CallEvents {
    hipEvent_t e[65];
    int n = 0;
    bool make(int count) {
        for (; n < count; ++n)
            if (hipEventCreateWithFlags(&e[n], hipEventDisableTiming) != hipSuccess) return false;
        return true;
    }
    ~CallEvents() {
        for (int i = 0; i < n; ++i) hipEventDestroy(e[i]);
    }
};

static csa_status index_attend_args(const char* fn, csa_dtype dt, int64_t B, int64_t Tq,
                                    int64_t H, int64_t D, int64_t HI, int64_t dI, int64_t Nc,
                                    int64_t m, int64_t W, int64_t k, int64_t q_pos0, float scale,
                                    const void* q, const void* q_idx, const uint8_t* k_codes,
                                    const uint8_t* k_scales, const void* ck, const void* cv,
                                    const void* rk, const void* rv, int64_t raw_pos0,
                                    int64_t raw_len, int32_t* topk, void* o, int64_t n_chunks) {
    CHECK(n_chunks >= 1 && n_chunks <= 64, CSA_EINVAL, "%s: n_chunks must be in [1, 64]", fn);
    // every check of the two steps over the whole range (workspaces apart)
    void* fake_ws = (void*)(uintptr_t)256;
    csa_status s = index_topk_do(false, fn, dt, B, Tq, HI, dI, Nc, m, W, k, q_pos0,
                                 dense_in(q_idx, Tq, HI * dI), k_codes, k_scales, topk, fake_ws,
                                 SIZE_MAX, nullptr);
    if (s == CSA_OK)
        s = csa_attend_do(false, fn, dt, B, Tq, H, D, Nc, m, W, k, q_pos0, scale,
                          dense_in(q, Tq, H * D), dense_in(ck, Nc, D), dense_in(cv, Nc, D), topk,
                          dense_in(rk, raw_len, D), dense_in(rv, raw_len, D), raw_pos0, raw_len,
                          dense_out(o, Tq, H * D), fake_ws, SIZE_MAX, nullptr);
    return s;
}

csa_status csa_index_attend_workspace(csa_dtype dt, int64_t B, int64_t Tq, int64_t H, int64_t D,
                                      int64_t HI, int64_t dI, int64_t Nc, int64_t m, int64_t W,
                                      int64_t k, int64_t q_pos0, int64_t n_chunks,
                                      size_t* bytes) {
    const char* fn = "csa_index_attend_workspace";
    CHECK(bytes, CSA_EINVAL, "%s: null pointer", fn);
    CHECK(n_chunks >= 1 && n_chunks <= 64, CSA_EINVAL, "%s: n_chunks must be in [1, 64]", fn);
    if (csa_status s = check_dtype(dt, fn)) return s;
    if (csa_status s = index_args(fn, B, Tq, HI, dI, Nc, m, W, k, q_pos0)) return s;
    if (csa_status s = attend_shape(fn, dt, B, Tq, H, D)) return s;
    const SliceWs w = slice_ws(dt, B, Tq, H, D, HI, dI, Nc, m, W, k, q_pos0, n_chunks);
    *bytes = align256(w.index) + w.attend;
    return ok();
}

csa_status csa_index_attend(csa_dtype dt, int64_t B, int64_t Tq, int64_t H, int64_t D,
                            int64_t HI, int64_t dI, int64_t Nc, int64_t m, int64_t W, int64_t k,
                            int64_t q_pos0, float scale, const void* q, const void* q_idx,
                            const uint8_t* k_codes, const uint8_t* k_scales, const void* ck,
                            const void* cv, const void* rk, const void* rv, int64_t raw_pos0,
                            int64_t raw_len, int32_t* topk, void* o, int64_t n_chunks, void* ws,
                            size_t ws_bytes, hipStream_t stream, hipStream_t aux_stream) {
    const char* fn = "csa_index_attend";
    if (csa_status s = index_attend_args(fn, dt, B, Tq, H, D, HI, dI, Nc, m, W, k, q_pos0, scale,
                                         q, q_idx, k_codes, k_scales, ck, cv, rk, rv, raw_pos0,
                                         raw_len, topk, o, n_chunks))
        return s;
    const SliceWs w = slice_ws(dt, B, Tq, H, D, HI, dI, Nc, m, W, k, q_pos0, n_chunks);
    const size_t need = align256(w.index) + w.attend;
    CHECK(ws_bytes >= need && (need == 0 || (ws && aligned16(ws))), CSA_EINVAL,
          "%s: workspace of %zu bytes given, %zu needed", fn, ws_bytes, need);
    if (B == 0 || Tq == 0) return ok();
    void* iws = ws;
    void* aws = w.attend ? (void*)((char*)ws + align256(w.index)) : nullptr;
    const bool two = aux_stream != stream;
    const int64_t per = (Tq + n_chunks - 1) / n_chunks;   // rows per slice
    const int n_slices = (int)((Tq + per - 1) / per);
    // events of this call (one per slice, one for the start), made here and
    // destroyed on return: a destroyed event that is still pending is
    // released by the runtime once it completes, and the waits already
    // queued on it stand
    CallEvents ev;
    const int n_ev = two ? n_slices + 1 : 0;
    if (!ev.make(n_ev)) return fail(CSA_EDEVICE, "%s: hipEventCreate failed", fn);
    hipStream_t is = two ? aux_stream : stream;
    if (two) {
        // the selection stream starts after everything already queued on stream
        if (hipEventRecord(ev.e[n_ev - 1], stream) != hipSuccess ||
            hipStreamWaitEvent(is, ev.e[n_ev - 1], 0) != hipSuccess)
            return fail(CSA_EDEVICE, "%s: stream ordering failed", fn);
    }
    const int64_t esz = dt == CSA_F32 ? 4 : 2;
    const char* qb = (const char*)q;
    const char* qib = (const char*)q_idx;
    char* ob = (char*)o;
    for (int64_t b = 0; b < B; ++b) {
        const char* ckb = (const char*)ck + b * Nc * D * esz;
        const char* cvb = (const char*)cv + b * Nc * D * esz;
        const char* rkb = (const char*)rk + b * raw_len * D * esz;
        const char* rvb = (const char*)rv + b * raw_len * D * esz;
        const uint8_t* kcb = k_codes + b * Nc * (dI / 2);
        const uint8_t* ksb = k_scales + b * Nc * (dI / 32);
        int c = 0;
        for (int64_t a = 0; a < Tq; a += per, ++c) {
            const int64_t rows = Tq - a < per ? Tq - a : per;
            const int64_t r0 = b * Tq + a;
            hipError_t e = csa::launch_index_topk(
                (int)dt, csa::plan_index(1, rows, (int)HI, (int)dI, Nc, m, W, (int)k, q_pos0 + a),
                1, rows, (int)HI, (int)dI, Nc, m, W, (int)k, q_pos0 + a, qib + r0 * HI * dI * esz,
                csa::RowStrides{Tq * HI * dI, HI * dI}, kcb, ksb, topk + r0 * k, iws, is);
            if (e == hipSuccess && two) e = hipEventRecord(ev.e[c], is);
            if (e != hipSuccess) return launched(e, fn);
        }
        c = 0;
        for (int64_t a = 0; a < Tq; a += per, ++c) {
            const int64_t rows = Tq - a < per ? Tq - a : per;
            const int64_t r0 = b * Tq + a;
            hipError_t e = two ? hipStreamWaitEvent(stream, ev.e[c], 0) : hipSuccess;
            if (e == hipSuccess)
                e = csa::launch_attend(
                    (int)dt, slice_attend_plan(dt, B, Tq, rows, H, D, k, W), 1, rows, H, D, Nc, m,
                    W, k, q_pos0 + a, scale,
                    attend_io(dense_in(qb + r0 * H * D * esz, Tq, H * D), dense_in(ckb, Nc, D),
                              dense_in(cvb, Nc, D), dense_in(rkb, raw_len, D),
                              dense_in(rvb, raw_len, D),
                              dense_out(ob + r0 * H * D * esz, Tq, H * D)),
                    topk + r0 * k, raw_pos0, raw_len, aws, stream);
            if (e != hipSuccess) return launched(e, fn);
        }
    }
    return ok();
}

// ---- a stack of layers ------------------------------------------------------

csa_status csa_layer_schedule(int64_t n_layers, int32_t* kinds) {
    const char* fn = "csa_layer_schedule";
    CHECK(n_layers >= 0 && n_layers <= 4096, CSA_EINVAL, "%s: n_layers must be in [0, 4096]", fn);
    CHECK(kinds || n_layers == 0, CSA_EINVAL, "%s: null pointer", fn);
    for (int64_t l = 0; l < n_layers; ++l)
        kinds[l] = l < 2 ? CSA_LAYER_HCA : (l % 2 == 0 ? CSA_LAYER_CSA : CSA_LAYER_HCA);
    return ok();
}

// workspace of one layer (the stack reuses one buffer, layer after layer)
static size_t layer_ws(csa_dtype dt, const csa_layer_desc& L, int64_t B, int64_t Tq, int64_t H,
                       int64_t D, int64_t HI, int64_t dI, int64_t W, int64_t k, int64_t q_pos0) {
    if (L.kind == CSA_LAYER_HCA)
        return csa::plan_attend((int)dt, B, Tq, H, D, hca_max_keys(Tq, L.m, W, q_pos0)).ws_bytes;
    const size_t a = csa::plan_attend((int)dt, B, Tq, H, D, k + W).ws_bytes;
    const size_t i = csa::plan_index(B, Tq, (int)HI, (int)dI, L.Nc, L.m, W, (int)k, q_pos0).ws_bytes;
    return a > i ? a : i;
}

static csa_status stack_args(const char* fn, csa_dtype dt, int64_t n_layers,
                             const csa_layer_desc* layers, int64_t B, int64_t Tq, int64_t H,
                             int64_t D, int64_t HI, int64_t dI, int64_t W, int64_t k,
                             int64_t q_pos0) {
    if (csa_status s = attend_shape(fn, dt, B, Tq, H, D)) return s;
    CHECK(n_layers >= 0 && n_layers <= 4096, CSA_EINVAL, "%s: n_layers must be in [0, 4096]", fn);
    CHECK(layers || n_layers == 0, CSA_EINVAL, "%s: null pointer", fn);
    for (int64_t l = 0; l < n_layers; ++l) {
        const csa_layer_desc& L = layers[l];
        CHECK(L.kind == CSA_LAYER_CSA || L.kind == CSA_LAYER_HCA, CSA_EINVAL,
              "%s: layer %lld: unknown kind %d", fn, (long long)l, (int)L.kind);
        csa_status s = L.kind == CSA_LAYER_CSA
                           ? index_args(fn, B, Tq, HI, dI, L.Nc, L.m, W, k, q_pos0)
                           : check_positions(fn, Tq, L.Nc, L.m, W, q_pos0, 0, -1);
        if (s != CSA_OK) {
            char inner[512];
            snprintf(inner, sizeof(inner), "%s", g_err);
            return fail(s, "layer %lld: %s", (long long)l, inner);
        }
    }
    return CSA_OK;
}

csa_status csa_stack_workspace(csa_dtype dt, int64_t n_layers, const csa_layer_desc* layers,
                               int64_t B, int64_t Tq, int64_t H, int64_t D, int64_t HI,
                               int64_t dI, int64_t W, int64_t k, int64_t q_pos0, size_t* bytes) {
    const char* fn = "csa_stack_workspace";
    CHECK(bytes, CSA_EINVAL, "%s: null pointer", fn);
    if (csa_status s = stack_args(fn, dt, n_layers, layers, B, Tq, H, D, HI, dI, W, k, q_pos0))
        return s;
    size_t need = 0;
    for (int64_t l = 0; l < n_layers; ++l) {
        const size_t n = layer_ws(dt, layers[l], B, Tq, H, D, HI, dI, W, k, q_pos0);
        need = n > need ? n : need;
    }
    *bytes = need;
    return ok();
}

// every layer is checked before the first launch
static csa_status stack_layer(bool run, const char* fn, int64_t l, csa_dtype dt,
                              const csa_layer_desc& L, int64_t B, int64_t Tq, int64_t H,
                              int64_t D, int64_t HI, int64_t dI, int64_t W, int64_t k,
                              int64_t q_pos0, float scale, int64_t raw_pos0, int64_t raw_len,
                              void* ws, size_t ws_bytes, hipStream_t stream) {
    csa_status s;
    if (L.kind == CSA_LAYER_CSA) {
        s = index_topk_do(run, "csa_index_topk", dt, B, Tq, HI, dI, L.Nc, L.m, W, k, q_pos0,
                          dense_in(L.q_idx, Tq, HI * dI), L.k_codes, L.k_scales, L.topk, ws,
                          ws_bytes, stream);
        if (s == CSA_OK)
            s = csa_attend_do(run, "csa_attend", dt, B, Tq, H, D, L.Nc, L.m, W, k, q_pos0, scale,
                              dense_in(L.q, Tq, H * D), dense_in(L.ck, L.Nc, D),
                              dense_in(L.cv, L.Nc, D), L.topk, dense_in(L.rk, raw_len, D),
                              dense_in(L.rv, raw_len, D), raw_pos0, raw_len,
                              dense_out(L.o, Tq, H * D), ws, ws_bytes, stream);
    } else {
        s = hca_attend_do(run, "hca_attend", dt, B, Tq, H, D, L.Nc, L.m, W, q_pos0, scale,
                          dense_in(L.q, Tq, H * D), dense_in(L.ck, L.Nc, D),
                          dense_in(L.cv, L.Nc, D), dense_in(L.rk, raw_len, D),
                          dense_in(L.rv, raw_len, D), raw_pos0, raw_len,
                          dense_out(L.o, Tq, H * D), ws, ws_bytes, stream);
    }
    if (s != CSA_OK) {
        char inner[512];
        snprintf(inner, sizeof(inner), "%s", g_err);
        return fail(s, "%s: layer %lld: %s", fn, (long long)l, inner);
    }
    return CSA_OK;
}

csa_status csa_stack_attend(csa_dtype dt, int64_t n_layers, const csa_layer_desc* layers,
                            int64_t B, int64_t Tq, int64_t H, int64_t D, int64_t HI, int64_t dI,
                            int64_t W, int64_t k, int64_t q_pos0, float scale, int64_t raw_pos0,
                            int64_t raw_len, void* ws, size_t ws_bytes, hipStream_t stream) {
    const char* fn = "csa_stack_attend";
    if (csa_status s = stack_args(fn, dt, n_layers, layers, B, Tq, H, D, HI, dI, W, k, q_pos0))
        return s;
    for (int pass = 0; pass < 2; ++pass)
        for (int64_t l = 0; l < n_layers; ++l)
            if (csa_status s = stack_layer(pass == 1, fn, l, dt, layers[l], B, Tq, H, D, HI, dI,
                                           W, k, q_pos0, scale, raw_pos0, raw_len, ws, ws_bytes,
                                           stream))
                return s;
    return ok();
}

csa_status csa_quantize_mxfp8(csa_dtype dt, int64_t rows, int64_t d, const void* x, void* codes,
                              void* scales, hipStream_t stream) {
    const char* fn = "csa_quantize_mxfp8";
    if (csa_status s = check_dtype(dt, fn)) return s;
    CHECK(rows >= 0, CSA_EINVAL, "%s: rows must be >= 0", fn);
    CHECK(d >= 32 && d % 32 == 0 && d <= 65536, CSA_EINVAL,
          "%s: d must be a multiple of 32 in [32, 65536] (got %lld)", fn, (long long)d);
    if (rows == 0) return ok();
    CHECK(x && codes && scales, CSA_EINVAL, "%s: null pointer", fn);
    CHECK(aligned16(x) && aligned16(codes), CSA_EINVAL, "%s: x and codes must be 16-byte aligned",
          fn);
    return launched(csa::launch_quant_mxfp8((int)dt, x, (uint8_t*)codes, (uint8_t*)scales, rows,
                                            (int)d, stream),
                    fn);
}

// Compressed entries as MXFP8: bf16 queries, window and output; D = 128.
static csa_status mx8_args(const char* fn, int64_t B, int64_t Tq, int64_t H, int64_t D,
                           const void* q, const void* ck, const void* cv, const void* cks,
                           const void* cvs, const void* rk, const void* rv, const void* o) {
    if (csa_status s = attend_shape(fn, CSA_BF16, B, Tq, H, D)) return s;
    CHECK(D == 128, CSA_EUNSUPPORTED, "%s: MXFP8 entries need D = 128", fn);
    CHECK(q && ck && cv && cks && cvs && rk && rv && o, CSA_EINVAL, "%s: null pointer", fn);
    CHECK(aligned16(q) && aligned16(ck) && aligned16(cv) && aligned16(rk) && aligned16(rv) &&
              aligned16(o), CSA_EINVAL, "%s: tensors must be 16-byte aligned", fn);
    CHECK(((uintptr_t)cks & 3u) == 0 && ((uintptr_t)cvs & 3u) == 0, CSA_EINVAL,
          "%s: scale tensors must be 4-byte aligned", fn);
    return CSA_OK;
}

csa_status csa_attend_mxfp8(int64_t B, int64_t Tq, int64_t H, int64_t D, int64_t Nc, int64_t m,
                            int64_t W, int64_t k, int64_t q_pos0, float scale, const void* q,
                            const void* ck, const void* cv, const void* ck_scales,
                            const void* cv_scales, const int32_t* topk, const void* rk,
                            const void* rv, int64_t raw_pos0, int64_t raw_len, void* o, void* ws,
                            size_t ws_bytes, hipStream_t stream) {
    const char* fn = "csa_attend_mxfp8";
    if (csa_status s = mx8_args(fn, B, Tq, H, D, q, ck, cv, ck_scales, cv_scales, rk, rv, o))
        return s;
    CHECK(topk, CSA_EINVAL, "%s: null pointer", fn);
    CHECK(k >= 1 && k <= 2048, CSA_EINVAL, "%s: k must be in [1, 2048]", fn);
    CHECK(raw_len >= 0, CSA_EINVAL, "%s: raw_len must be >= 0", fn);
    if (csa_status s = check_positions(fn, Tq, Nc, m, W, q_pos0, raw_pos0, raw_len)) return s;
    if (csa_status s = attend_ranges(fn, Nc, D, raw_len, k, W, q_pos0, Tq, m)) return s;
    csa::AttendPlan p = csa::plan_attend(1, B, Tq, H, D, k + W);
    CHECK(ws_bytes >= p.ws_bytes && (p.ws_bytes == 0 || (ws && aligned16(ws))), CSA_EINVAL,
          "%s: workspace of %zu bytes given, %zu needed", fn, ws_bytes, p.ws_bytes);
    return launched(csa::launch_attend_mx8(
                        p, B, Tq, H, Nc, m, W, k, q_pos0, scale,
                        attend_io(dense_in(q, Tq, H * D), dense_in(ck, Nc, D),
                                  dense_in(cv, Nc, D), dense_in(rk, raw_len, D),
                                  dense_in(rv, raw_len, D), dense_out(o, Tq, H * D)),
                        (const uint8_t*)ck_scales, (const uint8_t*)cv_scales, topk, raw_pos0,
                        raw_len, ws, stream),
                    fn);
}

csa_status hca_attend_mxfp8(int64_t B, int64_t Tq, int64_t H, int64_t D, int64_t Nc, int64_t m,
                            int64_t W, int64_t q_pos0, float scale, const void* q, const void* ck,
                            const void* cv, const void* ck_scales, const void* cv_scales,
                            const void* rk, const void* rv, int64_t raw_pos0, int64_t raw_len,
                            void* o, void* ws, size_t ws_bytes, hipStream_t stream) {
    const char* fn = "hca_attend_mxfp8";
    if (csa_status s = mx8_args(fn, B, Tq, H, D, q, ck, cv, ck_scales, cv_scales, rk, rv, o))
        return s;
    CHECK(raw_len >= 0, CSA_EINVAL, "%s: raw_len must be >= 0", fn);
    if (csa_status s = check_positions(fn, Tq, Nc, m, W, q_pos0, raw_pos0, raw_len)) return s;
    if (csa_status s = attend_ranges(fn, Nc, D, raw_len, 0, W, q_pos0, Tq, m)) return s;
    csa::AttendPlan p = csa::plan_attend(1, B, Tq, H, D, hca_max_keys(Tq, m, W, q_pos0));
    CHECK(ws_bytes >= p.ws_bytes && (p.ws_bytes == 0 || (ws && aligned16(ws))), CSA_EINVAL,
          "%s: workspace of %zu bytes given, %zu needed", fn, ws_bytes, p.ws_bytes);
    return launched(csa::launch_attend_mx8(
                        p, B, Tq, H, Nc, m, W, 0, q_pos0, scale,
                        attend_io(dense_in(q, Tq, H * D), dense_in(ck, Nc, D),
                                  dense_in(cv, Nc, D), dense_in(rk, raw_len, D),
                                  dense_in(rv, raw_len, D), dense_out(o, Tq, H * D)),
                        (const uint8_t*)ck_scales, (const uint8_t*)cv_scales, nullptr, raw_pos0,
                        raw_len, ws, stream),
                    fn);
}

}  // extern "C"

// ---- FP8 arithmetic (one exponent per row) ------------------------------------

extern "C" {

csa_status csa_quantize_fp8_rows(csa_dtype dt, int64_t rows, int64_t d, const void* x,
                                 void* codes, void* scales, hipStream_t stream) {
    const char* fn = "csa_quantize_fp8_rows";
    if (csa_status s = check_dtype(dt, fn)) return s;
    CHECK(rows >= 0, CSA_EINVAL, "%s: rows must be >= 0", fn);
    CHECK(d == 32 || d == 64 || d == 128 || d == 256, CSA_EUNSUPPORTED,
          "%s: d must be 32, 64, 128 or 256 (got %lld)", fn, (long long)d);
    if (rows == 0) return ok();
    CHECK(x && codes && scales, CSA_EINVAL, "%s: null pointer", fn);
    CHECK(aligned16(x) && aligned16(codes), CSA_EINVAL, "%s: x and codes must be 16-byte aligned",
          fn);
    CHECK(((uintptr_t)scales & 3u) == 0, CSA_EINVAL, "%s: scales must be 4-byte aligned", fn);
    return launched(csa::launch_quant_fp8_rows((int)dt, x, (uint8_t*)codes, (uint32_t*)scales,
                                               rows, (int)d, stream),
                    fn);
}

}  // extern "C"

// bf16 queries and output, FP8 rows for every K/V source; D = 128.
static csa_status fp8_args(const char* fn, int64_t B, int64_t Tq, int64_t H, int64_t D,
                           const void* q, const void* ck, const void* cv, const void* cks,
                           const void* cvs, const void* rk, const void* rv, const void* rks,
                           const void* rvs, const void* o) {
    if (csa_status s = attend_shape(fn, CSA_BF16, B, Tq, H, D)) return s;
    CHECK(D == 128, CSA_EUNSUPPORTED, "%s: FP8 attention needs D = 128", fn);
    CHECK(q && ck && cv && cks && cvs && rk && rv && rks && rvs && o, CSA_EINVAL,
          "%s: null pointer", fn);
    CHECK(aligned16(q) && aligned16(ck) && aligned16(cv) && aligned16(rk) && aligned16(rv) &&
              aligned16(o), CSA_EINVAL, "%s: q, o and the code tensors must be 16-byte aligned",
          fn);
    CHECK(((uintptr_t)cks & 3u) == 0 && ((uintptr_t)cvs & 3u) == 0 &&
              ((uintptr_t)rks & 3u) == 0 && ((uintptr_t)rvs & 3u) == 0,
          CSA_EINVAL, "%s: scale tensors must be 4-byte aligned", fn);
    return CSA_OK;
}

static csa::Fp8IO fp8_io(const void* q, const void* ck, const void* cv, const void* cks,
                         const void* cvs, const void* rk, const void* rv, const void* rks,
                         const void* rvs, void* o) {
    return csa::Fp8IO{(const uint16_t*)q,  (const uint8_t*)ck,  (const uint8_t*)cv,
                      (const uint8_t*)cks, (const uint8_t*)cvs, (const uint8_t*)rk,
                      (const uint8_t*)rv,  (const uint8_t*)rks, (const uint8_t*)rvs,
                      (uint16_t*)o};
}

extern "C" {

csa_status csa_attend_fp8(int64_t B, int64_t Tq, int64_t H, int64_t D, int64_t Nc, int64_t m,
                          int64_t W, int64_t k, int64_t q_pos0, float scale, const void* q,
                          const void* ck, const void* cv, const void* ck_scales,
                          const void* cv_scales, const int32_t* topk, const void* rk,
                          const void* rv, const void* rk_scales, const void* rv_scales,
                          int64_t raw_pos0, int64_t raw_len, void* o, void* ws, size_t ws_bytes,
                          hipStream_t stream) {
    const char* fn = "csa_attend_fp8";
    if (csa_status s = fp8_args(fn, B, Tq, H, D, q, ck, cv, ck_scales, cv_scales, rk, rv,
                                rk_scales, rv_scales, o))
        return s;
    CHECK(topk, CSA_EINVAL, "%s: null pointer", fn);
    CHECK(k >= 1 && k <= 2048, CSA_EINVAL, "%s: k must be in [1, 2048]", fn);
    CHECK(raw_len >= 0, CSA_EINVAL, "%s: raw_len must be >= 0", fn);
    if (csa_status s = check_positions(fn, Tq, Nc, m, W, q_pos0, raw_pos0, raw_len)) return s;
    if (csa_status s = attend_ranges(fn, Nc, D, raw_len, k, W, q_pos0, Tq, m)) return s;
    csa::AttendPlan p = csa::plan_attend(1, B, Tq, H, D, k + W);
    CHECK(ws_bytes >= p.ws_bytes && (p.ws_bytes == 0 || (ws && aligned16(ws))), CSA_EINVAL,
          "%s: workspace of %zu bytes given, %zu needed", fn, ws_bytes, p.ws_bytes);
    return launched(csa::launch_attend_fp8(p, B, Tq, H, Nc, m, W, k, q_pos0, scale,
                                           fp8_io(q, ck, cv, ck_scales, cv_scales, rk, rv,
                                                  rk_scales, rv_scales, o),
                                           topk, raw_pos0, raw_len, ws, stream),
                    fn);
}

csa_status hca_attend_fp8(int64_t B, int64_t Tq, int64_t H, int64_t D, int64_t Nc, int64_t m,
                          int64_t W, int64_t q_pos0, float scale, const void* q, const void* ck,
                          const void* cv, const void* ck_scales, const void* cv_scales,
                          const void* rk, const void* rv, const void* rk_scales,
                          const void* rv_scales, int64_t raw_pos0, int64_t raw_len, void* o,
                          void* ws, size_t ws_bytes, hipStream_t stream) {
    const char* fn = "hca_attend_fp8";
    if (csa_status s = fp8_args(fn, B, Tq, H, D, q, ck, cv, ck_scales, cv_scales, rk, rv,
                                rk_scales, rv_scales, o))
        return s;
    CHECK(raw_len >= 0, CSA_EINVAL, "%s: raw_len must be >= 0", fn);
    if (csa_status s = check_positions(fn, Tq, Nc, m, W, q_pos0, raw_pos0, raw_len)) return s;
    if (csa_status s = attend_ranges(fn, Nc, D, raw_len, 0, W, q_pos0, Tq, m)) return s;
    csa::AttendPlan p = csa::plan_attend(1, B, Tq, H, D, hca_max_keys(Tq, m, W, q_pos0));
    CHECK(ws_bytes >= p.ws_bytes && (p.ws_bytes == 0 || (ws && aligned16(ws))), CSA_EINVAL,
          "%s: workspace of %zu bytes given, %zu needed", fn, ws_bytes, p.ws_bytes);
    return launched(csa::launch_attend_fp8(p, B, Tq, H, Nc, m, W, 0, q_pos0, scale,
                                           fp8_io(q, ck, cv, ck_scales, cv_scales, rk, rv,
                                                  rk_scales, rv_scales, o),
                                           nullptr, raw_pos0, raw_len, ws, stream),
                    fn);
}

}  // extern "C"
