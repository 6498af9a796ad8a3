// Drives every entry point of the C ABI on the host, with the kernel
// dispatchers replaced by stand-ins (dispatch_stubs.cpp), so that the
// argument checks and the size / workspace / layout arithmetic run under
// AddressSanitizer and UndefinedBehaviorSanitizer.  Device pointers are
// fake, 16-byte aligned addresses that nothing dereferences.  Exits 0 and
// prints "abi ok" when every expected status matched and no sanitizer fired.
#include <stdint.h>
#include <stdio.h>

#include <initializer_list>

#include "mamba_scan.h"

namespace mscan {
extern int g_dispatched;
}

namespace {

int g_fail = 0;
#define EXPECT(call, want)                                                              \
  do {                                                                                  \
    const int got_ = (int)(call);                                                       \
    if (got_ != (int)(want)) {                                                          \
      fprintf(stderr, "line %d: %s -> %d, expected %d\n", __LINE__, #call, got_, (int)(want)); \
      ++g_fail;                                                                         \
    }                                                                                   \
  } while (0)

float* const P = reinterpret_cast<float*>(uintptr_t(4096));   // aligned, never dereferenced
float* const Q = reinterpret_cast<float*>(uintptr_t(4100));   // misaligned
const uint8_t* const F = reinterpret_cast<const uint8_t*>(uintptr_t(8192));
const size_t BIG = SIZE_MAX;                                   // "enough" workspace

mamba_status fwd(int64_t b, int64_t d, int64_t n, int64_t l, mamba_dtype dt = MAMBA_F32,
                 mamba_disc disc = MAMBA_DISC_ZOH, void* ws = P, size_t wsb = BIG,
                 const uint8_t* rst = nullptr, int lanes = 0, int segs = 0, float* ck = nullptr) {
  return mamba_scan_fwd_ex(P, P, P, P, P, P, P, P, P, rst, 1, disc, dt, b, d, n, l, P, P, ws, wsb,
                           nullptr, lanes, segs, ck, nullptr, nullptr);
}

mamba_status bwd(int64_t b, int64_t d, int64_t n, int64_t l, mamba_dtype dt = MAMBA_F32,
                 void* ws = P, size_t wsb = BIG, const uint8_t* rst = nullptr, int lanes = 0,
                 const float* ck = nullptr, int segs = 0) {
  return mamba_scan_bwd_ex(P, P, P, P, P, P, P, P, P, P, rst, 1, MAMBA_DISC_ZOH, dt, b, d, n, l, P,
                           P, P, P, P, P, P, P, P, ws, wsb, nullptr, lanes, segs, ck, nullptr,
                           nullptr);
}

// Every query and call over one size tuple; the statuses only have to be
// valid codes (the sanitizers watch the arithmetic).
void sweep(int64_t b, int64_t d, int64_t n, int64_t l) {
  const mamba_dtype dts[] = {MAMBA_F32, MAMBA_BF16};
  for (mamba_dtype dt : dts) {
    for (int lanes : {0, 16, 32, 64}) {
      for (int segs : {0, 1, 2, 1000}) {
        (void)mamba_scan_fwd_workspace_size_ex(b, d, n, l, dt, lanes, segs);
        const int s = fwd(b, d, n, l, dt, MAMBA_DISC_ZOH, P, BIG, nullptr, lanes, segs);
        if (s < 0 || s > 8) ++g_fail;
      }
      for (int segs : {0, 1, 2, 1000}) {
        (void)mamba_scan_bwd_workspace_size_ex(b, d, n, l, dt, lanes, segs);
        const int s = bwd(b, d, n, l, dt, P, BIG, nullptr, lanes, nullptr, segs);
        if (s < 0 || s > 8) ++g_fail;
      }
    }
    (void)mamba_scan_fwd_workspace_size(b, d, n, l, dt);
    (void)mamba_scan_bwd_workspace_size(b, d, n, l, dt);
    (void)fwd(b, d, n, l, dt, MAMBA_DISC_EULER, P, BIG, F, 16, 0, P);
    (void)bwd(b, d, n, l, dt, P, BIG, F, 16, P);
    (void)mamba_state_update(P, P, P, P, P, P, P, P, P, 1, MAMBA_DISC_ZOH, dt, b, d, n, P,
                             nullptr);
    (void)mamba_state_update_complex(P, P, P, P, P, P, P, P, P, 1, MAMBA_DISC_ZOH, dt, b, d, n,
                                     P, nullptr);
    for (int segs : {0, 1, 3, 1000}) {
      (void)mamba_scan_fwd_complex_workspace_size_ex(b, d, n, l, segs);
      (void)mamba_scan_bwd_complex_workspace_size_ex(b, d, n, l, segs);
      (void)mamba_scan_fwd_complex_ex(P, P, P, P, P, P, P, P, P, F, 1, MAMBA_DISC_ZOH, dt, b, d, n,
                                      l, P, P, P, P, BIG, nullptr, segs);
      (void)mamba_scan_bwd_complex_ex(P, P, P, P, P, P, P, P, P, P, F, 1, MAMBA_DISC_ZOH, dt, b, d,
                                      n, l, P, P, P, P, P, P, P, P, P, nullptr, P, BIG, nullptr,
                                      segs);
    }
    for (int64_t w : {1, 4, 5})
      (void)mamba_conv1d_silu_fwd(P, P, P, F, w, dt, b, d, l, P, nullptr);
    (void)mamba_conv1d_silu_bwd(P, P, P, F, P, 4, dt, b, d, l, P, P, P, nullptr);
  }
  (void)mamba_scan_checkpoint_size(b, d, n, l);
  (void)mamba_scan_complex_checkpoint_size(b, d, n, l);
  (void)mamba_scan_bwd_complex_workspace_size(b, d, n, l);
  (void)mamba_scan_fwd_complex_workspace_size(b, d, n, l);
}

}  // namespace

int main() {
  EXPECT(mamba_abi_version(), 2);
  for (int s = -1; s <= 10; ++s)
    if (mamba_status_string((mamba_status)s) == nullptr) ++g_fail;

  // ---- the targeted cases (statuses as documented in the header) ----
  EXPECT(fwd(2, 64, 16, 2048), MAMBA_OK);
  EXPECT(fwd(0, 64, 16, 2048), MAMBA_ERR_SHAPE);
  EXPECT(fwd(2, 64, 65, 2048), MAMBA_ERR_UNSUPPORTED);
  EXPECT(fwd(2, 64, 16, 2048, (mamba_dtype)7), MAMBA_ERR_DTYPE);
  EXPECT(fwd(2, 64, 16, 2048, MAMBA_F32, (mamba_disc)3), MAMBA_ERR_DTYPE);
  EXPECT(fwd(2, 64, 16, 2048, MAMBA_F32, MAMBA_DISC_ZOH, P, BIG, nullptr, 64, 0, P),
         MAMBA_ERR_UNSUPPORTED);                                   // checkpoints need 16 lanes
  EXPECT(fwd(2, 64, 16, 2048, MAMBA_F32, MAMBA_DISC_ZOH, P, BIG, nullptr, 0, 0, Q),
         MAMBA_ERR_ALIGNMENT);
  EXPECT(mamba_scan_fwd(P, P, P, P, P, nullptr, nullptr, nullptr, nullptr, 1, MAMBA_DISC_ZOH,
                        MAMBA_F32, 2, 64, 16, 2048, nullptr, nullptr, P, BIG, nullptr),
         MAMBA_ERR_NULL_PTR);
  EXPECT(mamba_scan_fwd_varlen(P, P, P, P, P, nullptr, nullptr, nullptr, nullptr, nullptr, 1,
                               MAMBA_DISC_ZOH, MAMBA_F32, 1, 16, 4, 128, P, nullptr, nullptr, 0,
                               nullptr),
         MAMBA_ERR_NULL_PTR);
  const size_t bws = mamba_scan_bwd_workspace_size(2, 64, 16, 2048, MAMBA_F32);
  EXPECT(bwd(2, 64, 16, 2048, MAMBA_F32, P, bws), MAMBA_OK);
  const size_t bws1 = mamba_scan_bwd_workspace_size_ex(2, 64, 16, 2048, MAMBA_F32, 0, 1);
  EXPECT(bwd(2, 64, 16, 2048, MAMBA_F32, P, bws - 1), MAMBA_OK);   // automatic: one pass
  EXPECT(bwd(2, 64, 16, 2048, MAMBA_F32, P, bws1 - 1, nullptr, 0, nullptr, 1),
         MAMBA_ERR_WORKSPACE);
  EXPECT(bwd(2, 64, 16, 2048, MAMBA_F32, nullptr, 0), MAMBA_ERR_WORKSPACE);
  EXPECT(bwd(2, 64, 16, 2048, MAMBA_F32, Q, bws), MAMBA_ERR_ALIGNMENT);
  EXPECT(mamba_scan_bwd(P, P, P, P, P, P, P, P, nullptr, P, 1, MAMBA_DISC_ZOH, MAMBA_F32, 2, 64,
                        16, 2048, P, P, P, P, P, nullptr, P, P, nullptr, P, bws, nullptr),
         MAMBA_ERR_INVALID);                                       // D given without dD
  {
    // segmented backward: its own workspace; the automatic choice falls back
    // to one pass when given only the unsegmented size
    const size_t seg = mamba_scan_bwd_workspace_size(1, 16, 16, 65536, MAMBA_F32);
    const size_t one = mamba_scan_bwd_workspace_size_ex(1, 16, 16, 65536, MAMBA_F32, 0, 1);
    if (!(seg > one)) ++g_fail;
    EXPECT(bwd(1, 16, 16, 65536, MAMBA_F32, P, one), MAMBA_OK);
    EXPECT(bwd(1, 16, 16, 65536, MAMBA_F32, P, seg), MAMBA_OK);
    EXPECT(bwd(1, 16, 16, 65536, MAMBA_F32, P, one, nullptr, 0, nullptr, 8), MAMBA_ERR_WORKSPACE);
    EXPECT(bwd(1, 16, 16, 65536, MAMBA_F32, P, seg, nullptr, 0, nullptr, -1),
           MAMBA_ERR_UNSUPPORTED);
  }
  EXPECT(mamba_scan_complex_checkpoint_size(2, 64, 17, 2049), SIZE_MAX);
  EXPECT(mamba_scan_bwd_complex_ex(P, P, P, P, P, nullptr, nullptr, nullptr, nullptr, P, nullptr, 1,
                                   MAMBA_DISC_ZOH, MAMBA_F32, 2, 64, 16, 2048, P, P, P, P, P,
                                   nullptr, nullptr, nullptr, nullptr, P, nullptr, 0, nullptr,
                                   0),
         MAMBA_OK);                             // checkpoints, automatic: no workspace, one pass
  {
    // complex segments: explicit counts need their workspace
    const size_t fw = mamba_scan_fwd_complex_workspace_size_ex(1, 16, 16, 65536, 8);
    const size_t bw = mamba_scan_bwd_complex_workspace_size_ex(1, 16, 16, 65536, 8);
    if (!(fw > 0 && bw > fw)) ++g_fail;
    EXPECT(mamba_scan_fwd_complex_ex(P, P, P, P, P, nullptr, nullptr, nullptr, nullptr, nullptr, 1,
                                     MAMBA_DISC_ZOH, MAMBA_F32, 1, 16, 16, 65536, P, nullptr,
                                     nullptr, P, fw - 1, nullptr, 8),
           MAMBA_ERR_WORKSPACE);
    EXPECT(mamba_scan_fwd_complex_ex(P, P, P, P, P, nullptr, nullptr, nullptr, nullptr, nullptr, 1,
                                     MAMBA_DISC_ZOH, MAMBA_F32, 1, 16, 16, 65536, P, P, nullptr,
                                     P, fw, nullptr, 8),
           MAMBA_OK);
    EXPECT(mamba_scan_fwd_complex(P, P, P, P, P, nullptr, nullptr, nullptr, nullptr, 1,
                                  MAMBA_DISC_ZOH, MAMBA_F32, 1, 16, 16, 65536, P, nullptr,
                                  nullptr, 0, nullptr),
           MAMBA_OK);                           // automatic without the workspace: one pass
    EXPECT(mamba_scan_bwd_complex_ex(P, P, P, P, P, nullptr, nullptr, nullptr, nullptr, P, nullptr, 1,
                                     MAMBA_DISC_ZOH, MAMBA_F32, 1, 16, 16, 65536, P, P, P, P, P,
                                     nullptr, nullptr, nullptr, nullptr, nullptr, P, bw - 1,
                                     nullptr, 8),
           MAMBA_ERR_WORKSPACE);
    EXPECT(mamba_scan_bwd_complex_ex(P, P, P, P, P, nullptr, nullptr, nullptr, nullptr, P, nullptr, 1,
                                     MAMBA_DISC_ZOH, MAMBA_F32, 1, 16, 16, 65536, P, P, P, P, P,
                                     nullptr, nullptr, nullptr, nullptr, nullptr, P, bw, nullptr,
                                     -1),
           MAMBA_ERR_UNSUPPORTED);
  }
  EXPECT(mamba_conv1d_silu_fwd(P, P, nullptr, nullptr, 5, MAMBA_F32, 1, 8, 64, P, nullptr),
         MAMBA_ERR_UNSUPPORTED);
  EXPECT(mamba_state_update(P, P, P, P, P, P, nullptr, nullptr, nullptr, 1, MAMBA_DISC_ZOH,
                            MAMBA_F32, 4, 32, 16, P, nullptr),
         MAMBA_OK);

  // ---- sweep of sizes, edges and extremes ----
  const int64_t sizes[] = {-1, 0, 1, 2, 15, 16, 17, 127, 128, 129, 1000, 1 << 20,
                           (int64_t)1 << 31, (int64_t)1 << 40, (int64_t)1 << 62, INT64_MAX};
  const int64_t states[] = {-1, 0, 1, 16, 17, 64, 65, INT64_MAX};
  for (int64_t b : sizes)
    for (int64_t d : sizes)
      for (int64_t n : states)
        for (int64_t l : sizes) {
          if ((b > 4096 && d > 4096) || (b > 4096 && l > 4096) || (d > 4096 && l > 4096)) {
            // large products: only the extremes combined (keeps the sweep short)
            if (!((b == INT64_MAX || d == INT64_MAX || l == INT64_MAX) ||
                  (b == ((int64_t)1 << 62) || d == ((int64_t)1 << 62) || l == ((int64_t)1 << 62))))
              continue;
          }
          sweep(b, d, n, l);
        }

  if (mscan::g_dispatched == 0) ++g_fail;
  if (g_fail) {
    fprintf(stderr, "%d check(s) failed\n", g_fail);
    return 1;
  }
  printf("abi ok (%d dispatches reached)\n", mscan::g_dispatched);
  return 0;
}
