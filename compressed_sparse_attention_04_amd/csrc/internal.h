// internal.h -- launchers shared between the kernel files and the C ABI
// layer of libcsa.so.  Arguments are validated by the caller (api.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "common.h"

namespace csa {

// dt: 0 = fp32, 1 = bf16 (same values as csa_dtype)
// x [B][T][C] and gate [B][T][gc] rows, out [B][T/m][C] rows, at their strides
hipError_t launch_compress(int dt, const void* x, RowStrides xs, const void* gate, RowStrides gs,
                           void* out, RowStrides os, int64_t B, int64_t T, int C, int m, int gc,
                           hipStream_t st);

// one decode step of cache upkeep (see hca_append); *new_win_pos0 gets the
// window buffer's first position after the call
hipError_t launch_append(int dt, int64_t B, int64_t C, int64_t m, int64_t W, int64_t t,
                         int64_t win_pos0, int64_t wcap, int64_t gc, int64_t nc_cap,
                         const void* k_new, const void* v_new, const void* gk_new,
                         const void* gv_new, void* rk, void* rv, void* gk_blk, void* gv_blk,
                         void* ck, void* cv, int64_t* new_win_pos0, hipStream_t st);

// x rows at x_rs elements apart; codes and scales dense
hipError_t launch_quant_mxfp4(int dt, const void* x, int64_t x_rs, uint8_t* codes,
                              uint8_t* scales, int64_t rows, int d, hipStream_t st);

// Indexer paths: STREAM (one block per 8 query rows streams all their
// candidates), DECODE (<= 8 rows over a long context: chunked scoring to
// the workspace + one select block per row), CHUNK (chunk-local top-k lists
// + merge; any size).
enum IndexPath { IDX_STREAM = 0, IDX_DECODE = 1, IDX_CHUNK = 2 };

struct IndexPlan {
    int path;
    int qt;            // queries per tile (32 / HI)
    int ch;            // candidates per chunk
    int64_t n_qtiles;
    int64_t n_chunks;  // chunks covering the largest candidate count
    size_t ws_bytes;   // partial lists when n_chunks > 1
};
IndexPlan plan_index(int64_t B, int64_t Tq, int HI, int dI, int64_t Nc, int64_t m, int64_t W,
                     int k, int64_t q_pos0);
// q_idx rows (query tokens of [HI][dI]) at the strides qs; keys dense
hipError_t launch_index_topk(int dt, const IndexPlan& p, int64_t B, int64_t Tq, int HI, int dI,
                             int64_t Nc, int64_t m, int64_t W, int k, int64_t q_pos0,
                             const void* q_idx, RowStrides qs, const uint8_t* k_codes,
                             const uint8_t* k_scales, int32_t* topk, void* ws, hipStream_t st);

struct AttendPlan {
    int splits;        // key-list splits per query (1 = no combine pass)
    size_t ws_bytes;   // split partials
};
AttendPlan plan_attend(int dt, int64_t B, int64_t Tq, int64_t H, int64_t D, int64_t max_keys);

// Tensors of one attention call: pointers and element strides (Q and O rows
// are query tokens holding [H][D] contiguously; K and V rows are compressed
// entries or raw tokens of D contiguous elements).
struct AttendIO {
    const void *q, *ck, *cv, *rk, *rv;
    void* o;
    RowStrides qs, cks, cvs, rks, rvs, os;
};
// topk == nullptr selects every candidate (HCA)
hipError_t launch_attend(int dt, const AttendPlan& p, int64_t B, int64_t Tq, int64_t H,
                         int64_t D, int64_t Nc, int64_t m, int64_t W, int64_t k,
                         int64_t q_pos0, float scale, const AttendIO& io, const int32_t* topk,
                         int64_t raw_pos0, int64_t raw_len, void* ws, hipStream_t st);

// bf16 queries and window rows, compressed K/V rows as MXFP8 (E4M3 codes
// [Nc][128] and E8M0 scales [Nc][4], dense; io.ck / io.cv are the codes);
// D = 128, the plan of the bf16 kernel
hipError_t launch_attend_mx8(const AttendPlan& p, int64_t B, int64_t Tq, int64_t H, int64_t Nc,
                             int64_t m, int64_t W, int64_t k, int64_t q_pos0, float scale,
                             const AttendIO& io, const uint8_t* cks, const uint8_t* cvs,
                             const int32_t* topk, int64_t raw_pos0, int64_t raw_len, void* ws,
                             hipStream_t st);

hipError_t launch_quant_mxfp8(int dt, const void* x, uint8_t* codes, uint8_t* scales,
                              int64_t rows, int d, hipStream_t st);
// one scale per row of d values (d / 32 in {1, 2, 4, 8}): a 32-bit word per
// row holding the fp32 power of two 2^e
hipError_t launch_quant_fp8_rows(int dt, const void* x, uint8_t* codes, uint32_t* scales,
                                 int64_t rows, int d, hipStream_t st);

// merge of bf16 split partials (layout of plan_attend's workspace) into o
void launch_attend_combine(const void* ws, int64_t B, int64_t Tq, int H, int D, int splits,
                           void* o, RowStrides os, hipStream_t st);

// FP8 arithmetic: bf16 queries (encoded per head row inside), FP8 rows for
// compressed K/V and window K/V (E4M3 codes [rows][128] and one scale word
// per row [rows], the fp32 bits of 2^e, dense), bf16 output; D = 128, the
// plan of the bf16 kernel
struct Fp8IO {
    const uint16_t* q;
    const uint8_t *ck, *cv, *cks, *cvs, *rk, *rv, *rks, *rvs;
    uint16_t* o;
};
hipError_t launch_attend_fp8(const AttendPlan& p, int64_t B, int64_t Tq, int64_t H, int64_t Nc,
                             int64_t m, int64_t W, int64_t k, int64_t q_pos0, float scale,
                             const Fp8IO& io, const int32_t* topk, int64_t raw_pos0,
                             int64_t raw_len, void* ws, hipStream_t st);

}  // namespace csa
