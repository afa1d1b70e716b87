/* inputs.h -- context structures of the synthetic-input callbacks in
 * libattnres_inputs.so (tests and benchmarks only; no AttnRes arithmetic).
 * The Python side mirrors these layouts with ctypes. */
#ifndef ATTNRES_INPUTS_H
#define ATTNRES_INPUTS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int (*attnres_inputs_fn)(void* ctx, int l, const void* h, const void** v_out,
                                 void* stream);

/* Generated sublayer outputs: v_l = scales[l-1] * N(0,1) under (seed, role, l),
 * written to slots[l % 3], each a device [R, D] buffer. scales is a host array. */
typedef struct {
  uint64_t seed;
  uint32_t role;
  int32_t dtype;
  int64_t R;
  int64_t D;
  int32_t L;
  int32_t pad;
  const double* scales;
  void* slots[3];
} attnres_inputs_ring;

/* Records rows[0..nrows) of every h_l into rec[(l-1)][nrows][row_bytes], then
 * calls inner(inner_ctx, ...). rec and rows are device buffers. */
typedef struct {
  attnres_inputs_fn inner;
  void* inner_ctx;
  void* rec;
  const int64_t* rows;
  int64_t nrows;
  int64_t row_bytes;
  int32_t L;
  int32_t pad;
} attnres_inputs_recorder;

int attnres_inputs_fill_normal(void* dst, int dtype, int64_t rows, int64_t D,
                               const int64_t* row_ids, uint64_t seed, uint32_t role,
                               uint32_t layer, double scale, void* stream);
int attnres_inputs_gather_rows(void* dst, const void* src, const int64_t* row_ids, int64_t nrows,
                               int64_t row_bytes, void* stream);
int attnres_inputs_ring_sublayer(void* ctx, int l, const void* h, const void** v_out, void* stream);
int attnres_inputs_record_sublayer(void* ctx, int l, const void* h, const void** v_out,
                                   void* stream);

#ifdef __cplusplus
}
#endif

#endif
