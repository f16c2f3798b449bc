// Shared declarations of the library's host code (not part of the ABI).
#pragma once
#include "serq.h"

namespace serq {

serq_status fail(serq_status st, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();
serq_status check_format(int32_t fmt);
serq_status make_layout(int32_t d_in, int32_t d_out, int32_t r, int32_t fmt, serq_layout *L);
serq_status check_layout(const serq_layout *L);
serq_status act_bytes(int32_t M, int32_t d_in, int32_t fmt, size_t *xq, size_t *xs);

// Largest d_in the single-pass activation quantizer keeps in registers.
constexpr int kQuantMaxInReg = 16384;
// INT4 activations carry one running code sum per 128 columns; the quantizer
// keeps them in LDS, which bounds d_in for INT4 at 128 * kQuantMaxChunks.
constexpr int kQuantMaxChunks = 512;

}  // namespace serq
