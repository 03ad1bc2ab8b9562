// host_checks.cpp -- the host-only part of the C ABI: the thread-local status
// text (pagedkv_last_error) and the validation of block tables and lengths
// held in host memory (pagedkv_check_tables), which PAGEDKV_DEBUG=1 runs
// before every launch.  No HIP: this file also builds with a plain host
// compiler (the sanitizer build of the host code).
#include <cstdarg>
#include <cstdint>
#include <cstdio>

#include "errors.h"
#include "pagedkv.h"

namespace pkv {

namespace {
thread_local char g_err[512] = "";
}  // namespace

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

}  // namespace pkv

using pkv::fail;

extern "C" {

const char* pagedkv_last_error(void) { return pkv::g_err; }

int pagedkv_check_tables(const int32_t* block_tables, const int32_t* context_lens,
                         const int32_t* cu_lens, int32_t B, int32_t T,
                         int32_t max_blocks_per_seq, int32_t num_blocks, int32_t block_size,
                         int32_t kind) {
  if (B < 0 || T < 0 || max_blocks_per_seq <= 0 || num_blocks <= 0 || block_size <= 0)
    return fail(PKV_ERR_INVALID_ARG, "check: B, T must be >= 0 and the sizes > 0");
  if (kind != PKV_CHECK_READ && kind != PKV_CHECK_APPEND && kind != PKV_CHECK_PREFILL)
    return fail(PKV_ERR_INVALID_ARG, "check: unknown kind %d", kind);
  if (B > 0 && (!block_tables || !context_lens))
    return fail(PKV_ERR_INVALID_ARG, "check: null table or lengths");
  if (kind != PKV_CHECK_READ || cu_lens) {
    if (!cu_lens) {
      if (T != B)
        return fail(PKV_ERR_INVALID_ARG, "check: one new token per sequence needs T (%d) == B (%d)",
                    T, B);
    } else {
      if (cu_lens[0] != 0)
        return fail(PKV_ERR_INVALID_ARG, "check: prefix sums start at %d, not 0", cu_lens[0]);
      for (int32_t b = 0; b < B; ++b)
        if (cu_lens[b + 1] < cu_lens[b])
          return fail(PKV_ERR_INVALID_ARG, "check: prefix sums decrease at sequence %d", b);
      if (cu_lens[B] != T)
        return fail(PKV_ERR_INVALID_ARG, "check: prefix sums end at %d, not T = %d", cu_lens[B],
                    T);
    }
  }
  const int64_t cap = (int64_t)max_blocks_per_seq * block_size;
  for (int32_t b = 0; b < B; ++b) {
    const int32_t ctx = context_lens[b];
    if (ctx < 0 || ctx > cap)
      return fail(PKV_ERR_INVALID_ARG,
                  "check: sequence %d has context length %d outside [0, %lld] (table of %d "
                  "blocks of %d)",
                  b, ctx, (long long)cap, max_blocks_per_seq, block_size);
    const int32_t n = kind == PKV_CHECK_READ ? 0 : cu_lens ? cu_lens[b + 1] - cu_lens[b] : 1;
    if (kind == PKV_CHECK_APPEND && ctx < n)
      return fail(PKV_ERR_INVALID_ARG,
                  "check: sequence %d appends %d tokens but its length after the append is %d", b,
                  n, ctx);
    if (kind == PKV_CHECK_PREFILL && ctx < n)
      return fail(PKV_ERR_INVALID_ARG,
                  "check: sequence %d has %d query tokens but only %d cached tokens", b, n, ctx);
    const int64_t used = (ctx + (int64_t)block_size - 1) / block_size;
    const int32_t* row = block_tables + (int64_t)b * max_blocks_per_seq;
    for (int64_t j = 0; j < used; ++j)
      if (row[j] < 0 || row[j] >= num_blocks)
        return fail(PKV_ERR_INVALID_ARG,
                    "check: sequence %d, logical block %lld maps to physical block %d outside "
                    "[0, %d)",
                    b, (long long)j, row[j], num_blocks);
  }
  return PKV_OK;
}

}  // extern "C"
