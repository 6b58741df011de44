// Host-side check of the C ABI's argument validation and workspace planning,
// built with AddressSanitizer and UndefinedBehaviorSanitizer on the host code
// (device code is built as usual).  It makes no GPU call: every decode,
// projection and quantisation request below either fails validation before
// anything is launched or is a pure size query.  A seeded generator walks
// shapes around the documented limits (zero, negative, huge, ragged) and the
// program checks the invariants that hold for every answer:
//   - a workspace query answers 0 exactly when the same shape fails validation;
//   - the default split count is positive exactly when the shape is valid;
//   - an explicit split count never needs more workspace than a larger one;
//   - every status code has a string, and a failing call leaves a message.
#include <cinttypes>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "qsvd.h"

namespace {

uint64_t g_state = 0x9E3779B97F4A7C15ull;
uint64_t next() {
  g_state ^= g_state << 13;
  g_state ^= g_state >> 7;
  g_state ^= g_state << 17;
  return g_state;
}
template <typename T>
T pick(const T *v, int n) { return v[next() % n]; }

int g_fail = 0;
#define CHECK(cond, ...)                                   \
  do {                                                     \
    if (!(cond)) {                                         \
      std::fprintf(stderr, "CHECK failed: %s: ", #cond);   \
      std::fprintf(stderr, __VA_ARGS__);                   \
      std::fprintf(stderr, "\n");                          \
      ++g_fail;                                            \
    }                                                      \
  } while (0)

// a distinct non-null address with 256-byte alignment; never dereferenced on
// these paths (validation fails first)
void *fake(uintptr_t k) { return reinterpret_cast<void *>((uintptr_t(1) << 20) + 256 * k); }

}  // namespace

int main() {
  const int32_t bs[] = {-1, 0, 1, 2, 16, 17, 65535, 65536, 1 << 30};
  const int64_t Ls[] = {-5, 0, 1, 31, 32, 33, 8191, 8192, 16384, 1 << 20, int64_t(1) << 40, int64_t(1) << 62};
  const int32_t rs[] = {-32, 0, 16, 32, 96, 128, 256, 384, 512, 768, 1536, 2048, 2304, 2560, 3072, 4096, 4097, 8192};
  const int32_t hs[] = {-1, 0, 1, 4, 16, 32, 33, 40, 64, 256, 257};
  const int32_t ds[] = {-64, 0, 16, 32, 48, 64, 100, 128, 256};
  const int32_t dts[] = {-1, QSVD_F32, QSVD_BF16, QSVD_I8, QSVD_I4, 4, 99};
  const int32_t sps[] = {-1, 0, 1, 2, 3, 7, 16, 64, 1023, 1024, 1025, 1 << 30};

  int valid = 0;
  for (int it = 0; it < 40000; ++it) {
    // every other request draws each argument from the values the library
    // supports, so that valid shapes are visited as often as invalid ones
    const bool plausible = it % 2 == 0;
    const int32_t b = plausible ? pick(bs + 2, 4) : pick(bs, 9);
    const int32_t r = pick(rs, 18);
    const int32_t heads = plausible ? pick(hs + 2, 6) : pick(hs, 11);
    const int32_t d = plausible ? ((next() & 1) ? 64 : 128) : pick(ds, 9);
    const int64_t L = plausible ? pick(Ls + 2, 6) : pick(Ls, 12);
    const qsvd_dtype_t cdt = static_cast<qsvd_dtype_t>(plausible ? pick(dts + 1, 4) : pick(dts, 7));
    const int32_t splits = pick(sps, 12);
    const size_t ws = qsvd_decode_workspace_bytes(b, L, r, heads, d, cdt, splits);
    const int32_t dflt = qsvd_decode_default_splits(b, L, r, heads, d, cdt);
    const size_t ws0 = qsvd_decode_workspace_bytes(b, L, r, heads, d, cdt, 0);
    CHECK((ws0 > 0) == (dflt > 0), "b=%d L=%" PRId64 " r=%d heads=%d d=%d dt=%d: ws0=%zu splits=%d",
          b, L, r, heads, d, cdt, ws0, dflt);
    if (splits >= 0) CHECK((ws > 0) == (ws0 > 0), "splits=%d changes validity", splits);
    if (ws > 0) {
      ++valid;
      // the decode call with this workspace but a missing output must fail
      // validation (nothing is launched)
      const qsvd_status_t st = qsvd_decode_attn(fake(1), cdt == QSVD_F32 ? QSVD_F32 : QSVD_BF16, fake(2), cdt,
                                                (cdt == QSVD_I8 || cdt == QSVD_I4) ? static_cast<const float *>(fake(3)) : nullptr,
                                                cdt == QSVD_I4 ? 128 : 0, fake(4), fake(5), cdt == QSVD_F32 ? QSVD_F32 : QSVD_BF16,
                                                nullptr, nullptr, b, L, r, heads, d, 0.125f, splits, nullptr,
                                                cdt == QSVD_F32 ? QSVD_F32 : QSVD_BF16, fake(6), ws, nullptr);
      CHECK(st == QSVD_ERR_INVALID, "NULL output accepted (status %d)", st);
      CHECK(std::strlen(qsvd_last_error()) > 0, "no message for a failing call");
      // a short workspace is rejected
      const qsvd_status_t st2 = qsvd_decode_attn(fake(1), cdt == QSVD_F32 ? QSVD_F32 : QSVD_BF16, fake(2), cdt,
                                                 (cdt == QSVD_I8 || cdt == QSVD_I4) ? static_cast<const float *>(fake(3)) : nullptr,
                                                 cdt == QSVD_I4 ? 128 : 0, fake(4), fake(5), cdt == QSVD_F32 ? QSVD_F32 : QSVD_BF16,
                                                 nullptr, nullptr, b, L, r, heads, d, 0.125f, splits, fake(7),
                                                 cdt == QSVD_F32 ? QSVD_F32 : QSVD_BF16, fake(6), ws - 1, nullptr);
      CHECK(st2 == QSVD_ERR_WORKSPACE || st2 == QSVD_ERR_INVALID, "short workspace accepted (status %d)", st2);
      // more splits never need less workspace (up to the clip at the tile count)
      if (splits > 0 && splits < 1024) {
        const size_t ws_more = qsvd_decode_workspace_bytes(b, L, r, heads, d, cdt, splits + 1);
        CHECK(ws_more >= ws, "splits %d -> %d shrinks the workspace %zu -> %zu", splits, splits + 1, ws, ws_more);
      }
    } else {
      // an invalid shape fails the call itself with a message, whatever the buffers
      const qsvd_status_t st = qsvd_decode_attn(fake(1), QSVD_BF16, fake(2), cdt, nullptr, 0, fake(4), fake(5),
                                                QSVD_BF16, nullptr, nullptr, b, L, r, heads, d, 0.125f, splits,
                                                fake(7), QSVD_BF16, fake(6), size_t(1) << 40, nullptr);
      CHECK(st < 0, "invalid shape accepted (b=%d L=%" PRId64 " r=%d heads=%d d=%d dt=%d)", b, L, r, heads, d, cdt);
    }

    // explicit and per-head entry points: size queries plus a NULL-output call
    const size_t we = qsvd_decode_explicit_workspace_bytes(b, L, r, heads, d);
    if (we > 0) {
      const qsvd_status_t st = qsvd_decode_attn_explicit(fake(1), QSVD_BF16, fake(2), QSVD_BF16, fake(3), fake(4),
                                                         QSVD_BF16, b, L, r, heads, d, 0.088f, nullptr, nullptr,
                                                         nullptr, QSVD_BF16, fake(5), we, nullptr);
      CHECK(st == QSVD_ERR_INVALID, "explicit: NULL output accepted (status %d)", st);
    }
    const int32_t rk = pick(rs, 18) / 8, rv = pick(rs, 18) / 8;
    const size_t wh = qsvd_decode_headwise_workspace_bytes(b, L, heads, d, rk, rv, splits);
    if (wh > 0) {
      const qsvd_status_t st = qsvd_decode_attn_headwise(fake(1), QSVD_BF16, fake(2), QSVD_BF16, fake(3), fake(4),
                                                         QSVD_BF16, b, L, heads, d, rk, rv, 0.088f, nullptr,
                                                         nullptr, splits, nullptr, QSVD_BF16, fake(5), wh, nullptr);
      CHECK(st == QSVD_ERR_INVALID, "headwise: NULL output accepted (status %d)", st);
    }

    // quantiser and projection: only invalid requests (no launch)
    const int64_t M = L;
    const int32_t n = r;
    const qsvd_status_t sq = qsvd_quantize_latent(fake(1), cdt, M, n, pick(ds, 9), QSVD_I8, pick(hs, 11), nullptr,
                                                  static_cast<float *>(fake(2)), nullptr);
    CHECK(sq < 0 || M <= 0, "quantise with NULL codes accepted (M=%" PRId64 ")", M);
    const qsvd_status_t sp = qsvd_project(fake(1), cdt, static_cast<const float *>(fake(2)), M, n, fake(3), cdt,
                                          nullptr, pick(rs, 18), nullptr, QSVD_F32, nullptr);
    CHECK(sp < 0 || M <= 0, "project with NULL output accepted (M=%" PRId64 ")", M);
  }
  for (int s = -6; s <= 1; ++s) CHECK(qsvd_status_string(static_cast<qsvd_status_t>(s)) != nullptr, "status %d", s);
  CHECK(valid > 1000, "only %d valid decode shapes visited", valid);
  std::printf("abi_fuzz: %d valid decode shapes, %d failures\n", valid, g_fail);
  return g_fail == 0 ? 0 : 1;
}
