// Host-side layout of the contiguous param/grad buffer.
//
// llm-infra-atlas, "05 · grad/param buffer": section 4.1 (reverse definition order), section 4.2
// (64-element parameter-start alignment, bucket-end padding to lcm(dp,128) or
// lcm(dp,128,2^16)), section 4.3 (bucket_size in elements, default max(40M, 1M*dp), a bucket is
// closed once param_end - bucket_start reaches bucket_size) and section 5 (one zero-filled
// param_data / grad_data pair, each parameter a view [start, end)).
#include <cstdint>
#include <numeric>

#include "sharded_linear.h"

namespace {

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

int64_t lcm64(int64_t a, int64_t b) { return a / std::gcd(a, b) * b; }

}  // namespace

extern "C" int64_t sl_default_bucket_size(int64_t dp) {
  const int64_t by_dp = 1000000LL * dp;
  return by_dp > 40000000LL ? by_dp : 40000000LL;
}

extern "C" int64_t sl_bucket_divisor(int64_t dp, int32_t high_busbw) {
  if (dp <= 0) return 0;
  int64_t d = lcm64(dp, 128);
  if (high_busbw) d = lcm64(d, 65536);
  return d;
}

extern "C" int sl_layout_build(int32_t n, const int64_t* numel, int64_t param_align,
                               int64_t bucket_size, int64_t divisor, int64_t* start,
                               int64_t* end, int32_t* bucket_id, int32_t bucket_cap,
                               int64_t* bucket_offset, int64_t* bucket_numel,
                               int64_t* bucket_numel_unpadded, int32_t* n_buckets,
                               int64_t* total_numel) {
  if (n < 0 || param_align <= 0 || divisor <= 0 || bucket_cap < 0) return SL_EINVAL;
  if (!n_buckets || !total_numel) return SL_EINVAL;
  if (n > 0 && (!numel || !start || !end || !bucket_id)) return SL_EINVAL;
  if (bucket_cap > 0 && (!bucket_offset || !bucket_numel || !bucket_numel_unpadded))
    return SL_EINVAL;
  for (int32_t i = 0; i < n; ++i)
    if (numel[i] < 0) return SL_EINVAL;

  // Walk the parameters last-defined first.  `cursor` is the next free element; a bucket is
  // the run [bucket_begin, padded end) that closes when it has reached bucket_size.
  int64_t bucket_begin = 0, cursor = 0, last_end = 0;
  int32_t nb = 0;
  bool open = false;
  auto close_bucket = [&](int64_t param_end) {
    const int64_t padded = round_up(param_end, divisor);
    if (nb < bucket_cap) {
      bucket_offset[nb] = bucket_begin;
      bucket_numel[nb] = padded - bucket_begin;
      bucket_numel_unpadded[nb] = param_end - bucket_begin;
    }
    ++nb;
    bucket_begin = padded;
    cursor = padded;
    open = false;
  };
  for (int32_t i = n - 1; i >= 0; --i) {
    const int64_t s = round_up(cursor, param_align);
    const int64_t e = s + numel[i];
    start[i] = s;
    end[i] = e;
    bucket_id[i] = nb;
    open = true;
    last_end = e;
    cursor = e;
    if (bucket_size > 0 && e - bucket_begin >= bucket_size) close_bucket(e);
  }
  if (open) close_bucket(last_end);
  *n_buckets = nb;
  *total_numel = bucket_begin;
  return nb > bucket_cap ? SL_ECAPACITY : SL_OK;
}

extern "C" const char* sl_status_str(int status) {
  switch (status) {
    case SL_OK: return "SL_OK";
    case SL_EINVAL: return "SL_EINVAL: invalid argument (null pointer, negative extent or option)";
    case SL_EALIGN: return "SL_EALIGN: device pointer not 16-byte aligned";
    case SL_ESHAPE: return "SL_ESHAPE: unsupported extent (in/out multiple of 8, 32 for MXFP8; < 2^31)";
    case SL_EWORKSPACE: return "SL_EWORKSPACE: workspace missing or too small";
    case SL_EHIP: return "SL_EHIP: HIP launch error";
    case SL_ECAPACITY: return "SL_ECAPACITY: output array too small";
    default: return "unknown status";
  }
}
