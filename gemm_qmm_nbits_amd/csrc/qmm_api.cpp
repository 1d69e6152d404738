// Host runtime of the qmm library: argument checks, path dispatch, the up-front
// tiling tuner and the extern "C" entry points declared in include/qmm.h.
//
// Error state ([P2] hip-ep PR 1328, "What": clear the HIP error state before the
// launches): every compute entry point calls hipGetLastError() once on entry and
// returns hipGetLastError() after its launches.
//
// Tuning ([P1] hip-ep PR 1318, "What", commit 1: GEMV autotune timed on rotated
// cold weights, median of cold bursts; [P2] "What": the first call of a shape
// times every candidate up front -- one discarded round then timed rounds, least
// total time wins -- writing only scratch, never while the stream is captured,
// under a mutex).  Every candidate computes the same bits, so the choice only
// affects speed.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <tuple>
#include <vector>

#include "qmm.h"
#include "qmm_internal.h"
#include "qmm_skinny.h"
#include "qmm_qmoe.h"

using namespace qmm;

namespace {

constexpr int kMaxGemvM = 8;  // M above this takes the prefill (matrix-core) path

bool is_pow2_block(int b) { return b >= 16 && b <= 256 && (b & (b - 1)) == 0; }
// zero point when none is given: the middle code of unsigned codes, 0 for signed int8
float default_zp(int bits) { return bits == 8 ? 0.0f : (float)(1 << (bits - 1)); }
bool valid_dtype(int t) { return t == QMM_F32 || t == QMM_F16 || t == QMM_BF16; }
size_t dtype_size(int t) { return t == QMM_F32 ? 4 : 2; }
bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Codebook weights with a 16-bit output: from this M on, the skinny matrix-core kernel
// beats the fp32 GEMV (it dequantizes each weight once for up to 16 rows), and its fp16
// operand rounding stays far below the output's own rounding.  The exception is M = 4
// on at most kCbGemvM4Codes codes, where the GEMV's four-row form wins (measured on
// MI355X: 4096 x 1024 8.6 against 12.7 us, 4096 x 2048 9.3 against 14.1, 4096 x 4096
// 11.4 against 12.1; 4096 x 14336 25.6 against 22.4).  A rule of the shape only, so a
// shape's path, and its bits, never depend on the device.
constexpr int kCbSkinnyMinM = 4;
constexpr int64_t kCbGemvM4Codes = int64_t(1) << 24;
bool codebook_gemv_m4(int64_t M, int64_t K, int64_t N) { return M == 4 && N * K <= kCbGemvM4Codes; }

// Workspace of the matrix-core paths: A as fp16 rows of K rounded up to 64, the
// fp32 row scales of that cast, then the fp32 partial sums of a split reduction (each
// region starts on a 256-byte boundary).
struct MatrixWorkspace {
  size_t a16 = 0, rs = 0, part = 0, total = 0;
};

MatrixWorkspace matrix_workspace(int64_t M, int64_t K, int64_t N) {
  MatrixWorkspace w;
  const int64_t kp = (K + 63) / 64 * 64;
  w.a16 = 0;
  w.rs = ((size_t)M * (size_t)kp * 2 + 255) & ~size_t(255);
  w.part = w.rs + (((size_t)M * 4 + 255) & ~size_t(255));
  const int splits = prefill_splits(M, N, kp);
  w.total = w.part + (splits > 1 ? (size_t)splits * (size_t)M * (size_t)N * 4 : 0);
  return w;
}

size_t matrix_workspace_bytes(int64_t M, int64_t K, int64_t N) { return matrix_workspace(M, K, N).total; }

// Matrix-core operands of A: fp16 A is read in place when its rows can be (16-byte
// aligned, K a multiple of 8 for the skinny kernel, of 64 for the tile kernel);
// otherwise A is cast into the workspace with the per-row pre-scale.
hipError_t matrix_activations(PrefillArgs& p, const void* A, int a_type, bool skinny, void* workspace,
                              hipStream_t st) {
  const MatrixWorkspace w = matrix_workspace(p.M, p.K, p.N);
  uint8_t* ws = (uint8_t*)workspace;
  p.partials = (float*)(ws + w.part);
  if (a_type == QMM_F16 && aligned(A, 16) && p.K % (skinny ? 8 : 64) == 0) {
    p.A16 = (const uint16_t*)A;
    p.lda = p.K;
    p.row_scale = nullptr;
    return hipSuccess;
  }
  p.A16 = (const uint16_t*)(ws + w.a16);
  p.lda = p.Kp;
  p.row_scale = (const float*)(ws + w.rs);
  return launch_cast_pad_f16(A, a_type, p.M, p.K, p.Kp, (uint16_t*)(ws + w.a16), (float*)(ws + w.rs), st);
}

// Whether qmm_codebook4 takes a matrix-core path (A rounded to fp16 in the workspace).
bool codebook_on_matrix_cores(int64_t M, int64_t K, int64_t N, int block, int c_type) {
  if (M <= 0 || K <= 0 || N <= 0) return false;
  if (M > kMaxGemvM) return true;
  if (M < kCbSkinnyMinM || c_type == QMM_F32 || codebook_gemv_m4(M, K, N)) return false;
  const int64_t Kp = (K + 63) / 64 * 64;
  const int64_t nblk = ceil_div(K, block);
  return skinny_applies(M, N, Kp, block, nblk * block / 2, nblk);
}

int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return 256;
  }
  if (cus[dev] == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) {
      (void)hipGetLastError();
      v = 256;
    }
    cus[dev] = v;
  }
  return cus[dev];
}

bool env_flag(const char* name) {
  const char* v = std::getenv(name);
  return v && v[0] && std::strcmp(v, "0") != 0;
}

// ---------------------------------------------------------------------------
// Tuner state
// ---------------------------------------------------------------------------
enum { ENTRY_NBITS = 0, ENTRY_CODEBOOK = 1, ENTRY_QMOE_FC1 = 2, ENTRY_QMOE_FC2 = 3, ENTRY_QMOE_FUSED = 4,
       ENTRY_COUNT = 5 };

// GEMV candidates: rows of W per lane (v_dot8 and fp32 kernels), then the matrix-core
// form of the 2-bit GEMV (one group of 16 rows per wave).
constexpr int kGemvCandidates[] = {1, 2, 4, kGemvMxBase + 1};
constexpr int kNumGemvCandidates = 4;
constexpr int kNumGemvRowCandidates = 3;  // the rows-per-lane candidates come first

struct TunerState {
  std::mutex mu;
  int mode = -1;  // -1: not yet read from the environment
  int forced = 0;
  std::map<std::tuple<int, int64_t, int64_t, int64_t, int, int, int, int>, int> choice;
  int last_choice[ENTRY_COUNT] = {-1, -1, -1, -1, -1};
  // cold-rotation pool (library-owned device memory, allocated on first tuning)
  uint8_t* pool = nullptr;
  size_t pool_bytes = 0;
  size_t pool_cursor = 0;
  void* out_scratch = nullptr;
  size_t out_scratch_bytes = 0;
};

TunerState& tuner() {
  static TunerState* t = new TunerState();  // lives until process end
  return *t;
}

int tuning_mode_locked(TunerState& t) {
  if (t.mode < 0) {
    t.mode = env_flag("QMM_NO_TUNE") ? 1 : 0;
    if (const char* f = std::getenv("QMM_FORCE_TILE")) {
      t.mode = 2;
      t.forced = std::atoi(f);
    }
  }
  return t.mode;
}

bool stream_capturing(hipStream_t st) {
  hipStreamCaptureStatus s = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(st, &s) != hipSuccess) {
    (void)hipGetLastError();
    return true;  // be conservative: do not time
  }
  return s != hipStreamCaptureStatusNone;
}

// Winner of an up-front timing: round 0 is discarded, the least total of the
// remaining rounds wins, ties go to the lower index.
int pick_winner(const double* t, int rounds, int ncand) {
  int best = 0;
  double best_total = 0;
  for (int c = 0; c < ncand; ++c) {
    double tot = 0;
    for (int r = 1; r < rounds; ++r) tot += t[r * ncand + c];
    if (c == 0 || tot < best_total) {
      best = c;
      best_total = tot;
    }
  }
  return best;
}

// The single-launch MoE forms (candidates 0 .. ncand - 2) against the two-kernel pair
// (candidate ncand - 1): the fastest single launch is kept unless the pair's total is
// more than kQmoePairMargin below it.  A second launch costs the host one more issue
// and the stream one more dependency, which the device-side timing does not see.
constexpr double kQmoePairMargin = 0.05;
int pick_single_launch(const double* t, int rounds, int ncand) {
  auto total = [&](int c) {
    double tot = 0;
    for (int r = 1; r < rounds; ++r) tot += t[r * ncand + c];
    return tot;
  };
  const int pair = ncand - 1;
  int best = -1;
  double best_total = 0;
  for (int c = 0; c < pair; ++c) {
    const double tot = total(c);
    if (best < 0 || tot < best_total) {
      best = c;
      best_total = tot;
    }
  }
  if (best < 0) return pair;
  return best_total <= total(pair) * (1.0 + kQmoePairMargin) ? best : pair;
}

// Ensure the rotation pool holds at least 4x the last-level cache (256 MB) and at
// least 4 copies of `unit` bytes.  Returns false when memory is not available.
bool ensure_pool(TunerState& t, size_t unit, size_t out_bytes) {
  const size_t want = std::max<size_t>(size_t(1) << 30, unit * 4);
  if (t.pool_bytes < want) {
    if (t.pool) (void)hipFree(t.pool);
    t.pool = nullptr;
    t.pool_bytes = 0;
    if (hipMalloc((void**)&t.pool, want) != hipSuccess) {
      (void)hipGetLastError();
      return false;
    }
    // deterministic content: every byte 0x5a (codes in range, scales finite)
    if (hipMemset(t.pool, 0x5a, want) != hipSuccess) {
      (void)hipGetLastError();
      return false;
    }
    t.pool_bytes = want;
    t.pool_cursor = 0;
  }
  if (t.out_scratch_bytes < out_bytes) {
    if (t.out_scratch) (void)hipFree(t.out_scratch);
    t.out_scratch = nullptr;
    t.out_scratch_bytes = 0;
    if (hipMalloc(&t.out_scratch, out_bytes) != hipSuccess) {
      (void)hipGetLastError();
      return false;
    }
    t.out_scratch_bytes = out_bytes;
  }
  return true;
}

// Give the rotation pool and the timing output back once a shape has been timed (the
// next new shape allocates them again); the timing has synchronized the stream.
void release_pool(TunerState& t) {
  if (t.pool) (void)hipFree(t.pool);
  if (t.out_scratch) (void)hipFree(t.out_scratch);
  (void)hipGetLastError();
  t.pool = nullptr;
  t.pool_bytes = 0;
  t.pool_cursor = 0;
  t.out_scratch = nullptr;
  t.out_scratch_bytes = 0;
}

// Next cold region of `unit` bytes in the pool (256-byte aligned).
uint8_t* next_region(TunerState& t, size_t unit) {
  const size_t u = (unit + 255) & ~size_t(255);
  if (t.pool_cursor + u > t.pool_bytes) t.pool_cursor = 0;
  uint8_t* p = t.pool + t.pool_cursor;
  t.pool_cursor += u;
  return p;
}

// Choose rows-per-lane for a GEMV shape, timing candidates on the first call.
int gemv_choice(int entry, const GemvArgs& g, hipStream_t st) {
  TunerState& t = tuner();
  std::lock_guard<std::mutex> lock(t.mu);
  const int mode = tuning_mode_locked(t);
  // default: the largest R that still gives >= 2 work-groups per compute unit
  auto default_idx = [&]() {
    const int subs = 64 >> g.lpr_log2;
    for (int i = kNumGemvRowCandidates - 1; i > 0; --i) {
      const int64_t tiles = ceil_div(g.N, 8LL * subs * kGemvCandidates[i]);
      if (tiles >= 2LL * g.num_cus) return i;
    }
    return 0;
  };
  if (mode == 2) {
    int f = t.forced;
    if (f < 0 || f >= kNumGemvCandidates) f = 0;
    t.last_choice[entry] = f;
    return kGemvCandidates[f];
  }
  if (mode == 1 || !g.chunked) {
    const int d = default_idx();
    t.last_choice[entry] = d;
    return kGemvCandidates[d];
  }
  const int64_t mb = g.M;  // M <= 8: one bucket per M
  auto key = std::make_tuple(entry, mb, g.K, g.N, g.bits, g.block, g.a_type, g.fmt);
  auto it = t.choice.find(key);
  if (it != t.choice.end()) {
    t.last_choice[entry] = it->second;
    return kGemvCandidates[it->second];
  }
  if (stream_capturing(st)) {  // no timing under capture: default now, decide later
    const int d = default_idx();
    t.last_choice[entry] = d;
    return kGemvCandidates[d];
  }
  // --- up-front cold timing -------------------------------------------------
  const size_t wbytes = (size_t)(g.N * g.row_bytes);
  const size_t sbytes = (size_t)(g.N * g.nblk) * (g.fmt == GEMV_CODEBOOK ? 4 : 2);
  const size_t zbytes = (g.zp_kind == QMM_ZP_PACKED) ? (size_t)(g.N * g.zp_row_bytes)
                        : (g.zp_kind == QMM_ZP_F16)  ? (size_t)(g.N * g.nblk * 2)
                                                     : 0;
  const size_t unit = ((wbytes + 255) & ~size_t(255)) + ((sbytes + 255) & ~size_t(255)) +
                      ((zbytes + 255) & ~size_t(255));
  const size_t obytes = (size_t)(g.M * g.N * 4);
  int chosen = default_idx();
  if (ensure_pool(t, unit, obytes)) {
    constexpr int kRounds = 9;
    constexpr int kBurst = 4;
    std::vector<double> times(kRounds * kNumGemvCandidates, 0.0);
    hipEvent_t e0, e1;
    bool ok = hipEventCreate(&e0) == hipSuccess && hipEventCreate(&e1) == hipSuccess;
    for (int r = 0; ok && r < kRounds; ++r) {
      for (int c = 0; ok && c < kNumGemvCandidates; ++c) {
        if (kGemvCandidates[c] > kGemvMxBase && !gemv_mx_supported(g)) {
          times[r * kNumGemvCandidates + c] = 1e30;  // not a form of this shape
          continue;
        }
        ok = hipEventRecord(e0, st) == hipSuccess;
        for (int b = 0; ok && b < kBurst; ++b) {
          GemvArgs tg = g;
          uint8_t* reg = next_region(t, unit);
          tg.W = reg;
          uint8_t* sp = reg + ((wbytes + 255) & ~size_t(255));
          if (g.fmt == GEMV_CODEBOOK) tg.absmax = (const float*)sp;
          else tg.scales = (const uint16_t*)sp;
          if (zbytes) tg.zp = sp + ((sbytes + 255) & ~size_t(255));
          tg.C = t.out_scratch;
          tg.c_type = QMM_F32;
          tg.bias = nullptr;
          ok = launch_gemv(tg, kGemvCandidates[c], st) == hipSuccess &&
               hipPeekAtLastError() == hipSuccess;
        }
        ok = ok && hipEventRecord(e1, st) == hipSuccess && hipEventSynchronize(e1) == hipSuccess;
        float ms = 0;
        ok = ok && hipEventElapsedTime(&ms, e0, e1) == hipSuccess;
        times[r * kNumGemvCandidates + c] = ms * 1000.0;
      }
    }
    if (ok) {
      chosen = pick_winner(times.data(), kRounds, kNumGemvCandidates);
      if (env_flag("QMM_LOG")) {
        std::fprintf(stderr, "[qmm] tune entry=%d M=%lld K=%lld N=%lld bits=%d block=%d ->", entry,
                     (long long)g.M, (long long)g.K, (long long)g.N, g.bits, g.block);
        for (int c = 0; c < kNumGemvCandidates; ++c) {
          double tot = 0;
          for (int r = 1; r < kRounds; ++r) tot += times[r * kNumGemvCandidates + c];
          std::fprintf(stderr, " R=%d:%.2fus", kGemvCandidates[c], tot / ((kRounds - 1) * kBurst));
        }
        std::fprintf(stderr, " pick R=%d\n", kGemvCandidates[chosen]);
      }
      t.choice[key] = chosen;
    } else {
      (void)hipGetLastError();  // timing failed: default tiling, decide again later
    }
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
  }
  release_pool(t);
  t.last_choice[entry] = chosen;
  return kGemvCandidates[chosen];
}

// MoE decode candidates, for fc1 and fc2 alike: rows per lane (low bits; an fc1 row
// is a g row and its u row) and the form (kQmoePerSlot: one work-group per row tile
// and slot; else the persistent form, fp mode only, with as many work-groups per
// compute unit as fit, or one with kQmoeOnePerCu).  All give the same bits.
constexpr int kQmoeCandidates[] = {1, 2, 1 | kQmoePerSlot, 2 | kQmoePerSlot, 1 | kQmoeOnePerCu,
                                   2 | kQmoeOnePerCu, 1 | kQmoeDedupe, 2 | kQmoeDedupe};
constexpr int kNumQmoeCandidates = 8;

struct QmoeTimingBufs {
  int32_t* ids = nullptr;  // timing expert ids, [kSets][T][k]
  size_t ids_count = 0;
  uint16_t* y = nullptr;   // timing output [T][H]
  size_t y_bytes = 0;
};

QmoeTimingBufs& qmoe_bufs() {
  static QmoeTimingBufs* b = new QmoeTimingBufs();
  return *b;
}

// Choose (fc1, fc2) rows-per-lane for a MoE shape.  The first uncaptured call of
// a shape times each candidate of each kernel: one discarded round, then 8 timed
// rounds, every timed launch on a different set of k experts (so the weights are
// read cold), writing only the call's scratch and a library-owned output.
void qmoe_choice(const QmoeArgs& a, hipStream_t st, bool may_time, int* r1, int* r2) {
  TunerState& t = tuner();
  std::lock_guard<std::mutex> lock(t.mu);
  const int mode = tuning_mode_locked(t);
  auto finish = [&](int c1, int c2) {
    t.last_choice[ENTRY_QMOE_FC1] = c1;
    t.last_choice[ENTRY_QMOE_FC2] = c2;
    *r1 = kQmoeCandidates[c1];
    *r2 = kQmoeCandidates[c2];
  };
  if (mode == 2) {
    int f = t.forced;
    if (f < 0 || f >= kNumQmoeCandidates * kNumQmoeCandidates) f = 0;
    finish(f % kNumQmoeCandidates, f / kNumQmoeCandidates);
    return;
  }
  if (mode == 1) {
    finish(0, 0);
    return;
  }
  auto key1 = std::make_tuple((int)ENTRY_QMOE_FC1, a.T * 1000 + a.k, a.H, a.I, a.block, a.mode,
                              (int)a.E, a.fc1.zp != nullptr);
  auto key2 = std::make_tuple((int)ENTRY_QMOE_FC2, a.T * 1000 + a.k, a.H, a.I, a.block, a.mode,
                              (int)a.E, a.fc2.zp != nullptr);
  auto i1 = t.choice.find(key1), i2 = t.choice.find(key2);
  if (i1 != t.choice.end() && i2 != t.choice.end()) {
    finish(i1->second, i2->second);
    return;
  }
  if (!may_time || stream_capturing(st)) {
    finish(0, 0);
    return;
  }
  QmoeTimingBufs& b = qmoe_bufs();
  constexpr int kRounds = 9;
  const int sets = kRounds * kNumQmoeCandidates * 2;
  const size_t ids_count = (size_t)sets * a.T * a.k;
  const size_t y_bytes = (size_t)a.T * a.H * 2;
  bool ok = true;
  if (b.ids_count < ids_count) {
    if (b.ids) (void)hipFree(b.ids);
    b.ids = nullptr;
    b.ids_count = 0;
    ok = hipMalloc((void**)&b.ids, ids_count * 4) == hipSuccess;
    if (ok) b.ids_count = ids_count;
  }
  if (ok && b.y_bytes < y_bytes) {
    if (b.y) (void)hipFree(b.y);
    b.y = nullptr;
    b.y_bytes = 0;
    ok = hipMalloc((void**)&b.y, y_bytes) == hipSuccess;
    if (ok) b.y_bytes = y_bytes;
  }
  int c1 = 0, c2 = 0;
  if (ok) {
    // timing expert sets: launch s of token tt uses experts (s*k*T + tt*k + j) mod E,
    // so consecutive launches touch different experts
    std::vector<int32_t> hid(ids_count);
    for (int s = 0; s < sets; ++s)
      for (int64_t tt = 0; tt < a.T; ++tt)
        for (int j = 0; j < a.k; ++j)
          hid[((size_t)s * a.T + tt) * a.k + j] =
              (int32_t)(((int64_t)s * a.k * a.T + tt * a.k + j) % a.E);
    ok = hipMemcpy(b.ids, hid.data(), ids_count * 4, hipMemcpyHostToDevice) == hipSuccess;
  }
  if (ok) {
    hipEvent_t e0, e1;
    ok = hipEventCreate(&e0) == hipSuccess && hipEventCreate(&e1) == hipSuccess;
    std::vector<double> t1(kRounds * kNumQmoeCandidates), t2(kRounds * kNumQmoeCandidates);
    int set = 0;
    for (int r = 0; ok && r < kRounds; ++r) {
      for (int which = 0; ok && which < 2; ++which) {
        for (int c = 0; ok && c < kNumQmoeCandidates; ++c) {
          QmoeArgs ta = a;
          ta.ids = b.ids + (size_t)(set++) * a.T * a.k;
          ta.Y = b.y;
          ok = hipEventRecord(e0, st) == hipSuccess;
          if (which == 0) ok = ok && launch_qmoe_fc1(ta, kQmoeCandidates[c], st) == hipSuccess;
          else ok = ok && launch_qmoe_fc2(ta, kQmoeCandidates[c], st) == hipSuccess;
          ok = ok && hipPeekAtLastError() == hipSuccess;
          ok = ok && hipEventRecord(e1, st) == hipSuccess && hipEventSynchronize(e1) == hipSuccess;
          float ms = 0;
          ok = ok && hipEventElapsedTime(&ms, e0, e1) == hipSuccess;
          (which == 0 ? t1 : t2)[r * kNumQmoeCandidates + c] = ms * 1000.0;
        }
      }
    }
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    if (ok) {
      c1 = pick_winner(t1.data(), kRounds, kNumQmoeCandidates);
      c2 = pick_winner(t2.data(), kRounds, kNumQmoeCandidates);
      t.choice[key1] = c1;
      t.choice[key2] = c2;
      if (env_flag("QMM_LOG")) {
        for (int which = 0; which < 2; ++which) {
          const std::vector<double>& tv = which == 0 ? t1 : t2;
          std::fprintf(stderr, "[qmm] tune qmoe fc%d T=%lld H=%lld I=%lld E=%lld k=%d block=%d mode=%d ->",
                       which + 1, (long long)a.T, (long long)a.H, (long long)a.I, (long long)a.E,
                       a.k, a.block, a.mode);
          for (int c = 0; c < kNumQmoeCandidates; ++c) {
            double tot = 0;
            for (int r = 1; r < kRounds; ++r) tot += tv[r * kNumQmoeCandidates + c];
            std::fprintf(stderr, " %s%d:%.2fus",
                         (kQmoeCandidates[c] & kQmoePerSlot)    ? "slot-R"
                         : (kQmoeCandidates[c] & kQmoeOnePerCu) ? "cu1-R"
                         : (kQmoeCandidates[c] & kQmoeDedupe)   ? "once-R"
                                                                : "R",
                         kQmoeCandidates[c] & 15, tot / (kRounds - 1));
          }
          std::fprintf(stderr, " pick #%d\n", which == 0 ? c1 : c2);
        }
      }
    }
  }
  if (!ok) {
    (void)hipGetLastError();
    c1 = c2 = 0;
  }
  finish(c1, c2);
}


// Candidate of the single-launch MoE form for a shape, or -1 for the two-kernel form
// with the tiling (r1, r2) already chosen by qmoe_choice.  The first uncaptured call of
// a shape times every single-launch candidate and that two-kernel pair the same way as
// qmoe_choice (one discarded round, then 8 timed rounds, every launch on a different
// expert set, writing only the call's scratch and a library-owned output), and
// pick_single_launch decides.  Without timing (tuning off, a first call under capture,
// the allocation-free entry) the single launch is used: candidate kQmoeDefaultFused
// (fc2 streamed, one work-group per compute unit) where its plan fits, else the
// two-kernel form.  Forced tuning: indices >= kQmoeForcedFused select candidate
// (index - kQmoeForcedFused) of the single-launch form, smaller ones the two-kernel form.
constexpr int kQmoeForcedFused = kNumQmoeCandidates * kNumQmoeCandidates;
constexpr int kQmoeDefaultFused = 1;

int qmoe_fused_choice(QmoeArgs& a, hipStream_t st, bool may_time, int r1, int r2) {
  TunerState& t = tuner();
  std::lock_guard<std::mutex> lock(t.mu);
  const int mode = tuning_mode_locked(t);
  auto plan = [&](int c) { return qmoe_fused_plan(a, c); };
  auto finish = [&](int c) {
    t.last_choice[ENTRY_QMOE_FUSED] = c;
    return c;
  };
  if (mode == 2) {
    if (t.forced < kQmoeForcedFused) return finish(-1);
    const int c = (t.forced - kQmoeForcedFused) % kNumQmoeFused;
    return plan(c) ? finish(c) : finish(-1);
  }
  auto untimed = [&] { return plan(kQmoeDefaultFused) ? finish(kQmoeDefaultFused) : finish(-1); };
  if (mode == 1) return untimed();
  auto key = std::make_tuple((int)ENTRY_QMOE_FUSED, a.T * 1000 + a.k, a.H, a.I, a.block, a.mode, (int)a.E,
                             (a.fc1.zp != nullptr ? 2 : 0) + (a.fc2.zp != nullptr ? 1 : 0));
  auto it = t.choice.find(key);
  if (it != t.choice.end()) return plan(it->second) ? finish(it->second) : finish(-1);
  if (!may_time || stream_capturing(st)) return untimed();
  bool any = false;
  for (int c = 0; c < kNumQmoeFused; ++c) any = any || plan(c);
  if (!any) {
    t.choice[key] = -1;
    return finish(-1);
  }
  QmoeTimingBufs& b = qmoe_bufs();
  constexpr int kRounds = 9;
  constexpr int kCands = kNumQmoeFused + 1;  // the last one is the two-kernel pair
  const int sets = kRounds * kCands;
  const size_t ids_count = (size_t)sets * a.T * a.k;
  const size_t y_bytes = (size_t)a.T * a.H * 2;
  bool ok = true;
  if (b.ids_count < ids_count) {
    if (b.ids) (void)hipFree(b.ids);
    b.ids = nullptr;
    b.ids_count = 0;
    ok = hipMalloc((void**)&b.ids, ids_count * 4) == hipSuccess;
    if (ok) b.ids_count = ids_count;
  }
  if (ok && b.y_bytes < y_bytes) {
    if (b.y) (void)hipFree(b.y);
    b.y = nullptr;
    b.y_bytes = 0;
    ok = hipMalloc((void**)&b.y, y_bytes) == hipSuccess;
    if (ok) b.y_bytes = y_bytes;
  }
  if (ok) {
    std::vector<int32_t> hid(ids_count);
    for (int s = 0; s < sets; ++s)
      for (int64_t tt = 0; tt < a.T; ++tt)
        for (int j = 0; j < a.k; ++j)
          hid[((size_t)s * a.T + tt) * a.k + j] = (int32_t)(((int64_t)s * a.k * a.T + tt * a.k + j) % a.E);
    ok = hipMemcpy(b.ids, hid.data(), ids_count * 4, hipMemcpyHostToDevice) == hipSuccess;
  }
  int best = kNumQmoeFused;
  if (ok) {
    hipEvent_t e0, e1;
    ok = hipEventCreate(&e0) == hipSuccess && hipEventCreate(&e1) == hipSuccess;
    std::vector<double> tv(kRounds * kCands, 1e30);
    int set = 0;
    for (int r = 0; ok && r < kRounds; ++r) {
      for (int c = 0; ok && c < kCands; ++c) {
        QmoeArgs ta = a;
        ta.ids = b.ids + (size_t)(set++) * a.T * a.k;
        ta.Y = b.y;
        if (c < kNumQmoeFused && !qmoe_fused_plan(ta, c)) continue;
        ok = hipEventRecord(e0, st) == hipSuccess;
        if (c < kNumQmoeFused) {
          ok = ok && launch_qmoe_fused(ta, st) == hipSuccess;
        } else {
          ok = ok && launch_qmoe_fc1(ta, r1, st) == hipSuccess && launch_qmoe_fc2(ta, r2, st) == hipSuccess;
        }
        ok = ok && hipPeekAtLastError() == hipSuccess;
        ok = ok && hipEventRecord(e1, st) == hipSuccess && hipEventSynchronize(e1) == hipSuccess;
        float ms = 0;
        ok = ok && hipEventElapsedTime(&ms, e0, e1) == hipSuccess;
        tv[r * kCands + c] = ms * 1000.0;
      }
    }
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    if (ok) {
      best = pick_single_launch(tv.data(), kRounds, kCands);
      t.choice[key] = best < kNumQmoeFused ? best : -1;
      if (env_flag("QMM_LOG")) {
        std::fprintf(stderr, "[qmm] tune qmoe fused T=%lld H=%lld I=%lld E=%lld k=%d block=%d ->", (long long)a.T,
                     (long long)a.H, (long long)a.I, (long long)a.E, a.k, a.block);
        for (int c = 0; c < kCands; ++c) {
          double tot = 0;
          for (int r = 1; r < kRounds; ++r) tot += tv[r * kCands + c];
          if (c < kNumQmoeFused)
            std::fprintf(stderr, " fc2R%d/w%d:%.2fus", kQmoeFusedR2[c % 2], kQmoeFusedWpc[c / 2], tot / (kRounds - 1));
          else
            std::fprintf(stderr, " two-kernel:%.2fus", tot / (kRounds - 1));
        }
        std::fprintf(stderr, " pick #%d\n", best);
      }
    }
  }
  if (!ok) {
    (void)hipGetLastError();
    best = kNumQmoeFused;
  }
  return (best < kNumQmoeFused && plan(best)) ? finish(best) : finish(-1);
}

// ---------------------------------------------------------------------------
// argument checks
// ---------------------------------------------------------------------------
qmm_status check_nbits(const void* A, int a_type, int64_t M, int64_t K, int64_t N, const uint8_t* W,
                       int bits, int block, const uint16_t* scales, const void* zp, int zp_kind,
                       const void* bias, const void* C, int c_type, const void* workspace,
                       size_t workspace_bytes) {
  (void)bias;
  if (!valid_dtype(a_type) || !valid_dtype(c_type)) return QMM_E_DTYPE;
  if (bits != 2 && bits != 3 && bits != 4 && bits != 8) return QMM_E_BITS;
  if (!is_pow2_block(block) || (bits == 3 && block < 32)) return QMM_E_BLOCK;
  if (M < 0 || K < 0 || N < 0 || M > (1LL << 30) || K > (1LL << 30) || N > (1LL << 30))
    return QMM_E_SHAPE;
  if (zp_kind < QMM_ZP_NONE || zp_kind > QMM_ZP_UNIFORM) return QMM_E_MODE;
  if (M == 0 || N == 0) return QMM_OK;
  if (!C) return QMM_E_NULL;
  if (K > 0 && (!A || !W || !scales)) return QMM_E_NULL;
  if ((zp_kind == QMM_ZP_PACKED || zp_kind == QMM_ZP_F16) && K > 0 && !zp) return QMM_E_NULL;
  if (!aligned(A, dtype_size(a_type)) || !aligned(C, dtype_size(c_type)) || !aligned(scales, 2))
    return QMM_E_ALIGN;
  if (bias && !aligned(bias, dtype_size(c_type))) return QMM_E_ALIGN;
  if (zp_kind == QMM_ZP_F16 && !aligned(zp, 2)) return QMM_E_ALIGN;
  const size_t need = qmm_nbits_workspace_bytes(M, K, N, a_type);
  if (need > 0 && (!workspace || workspace_bytes < need)) return QMM_E_WORKSPACE;
  if (need > 0 && !aligned(workspace, 16)) return QMM_E_ALIGN;
  return QMM_OK;
}

qmm_status check_codebook(const void* A, int a_type, int64_t M, int64_t K, int64_t N,
                          const uint8_t* W, int block, const float* absmax, const float* codebook,
                          const void* bias, const void* C, int c_type, const void* workspace,
                          size_t workspace_bytes) {
  if (!valid_dtype(a_type) || !valid_dtype(c_type)) return QMM_E_DTYPE;
  if (!is_pow2_block(block)) return QMM_E_BLOCK;
  if (M < 0 || K < 0 || N < 0 || M > (1LL << 30) || K > (1LL << 30) || N > (1LL << 30))
    return QMM_E_SHAPE;
  if (M == 0 || N == 0) return QMM_OK;
  if (!C) return QMM_E_NULL;
  if (K > 0 && (!A || !W || !absmax || !codebook)) return QMM_E_NULL;
  if (!aligned(A, dtype_size(a_type)) || !aligned(C, dtype_size(c_type)) || !aligned(absmax, 4) ||
      !aligned(codebook, 4))
    return QMM_E_ALIGN;
  if (bias && !aligned(bias, dtype_size(c_type))) return QMM_E_ALIGN;
  const size_t need = codebook_on_matrix_cores(M, K, N, block, c_type)
                          ? qmm_codebook4_workspace_bytes(M, K, N, a_type)
                          : 0;
  if (need > 0 && (!workspace || workspace_bytes < need)) return QMM_E_WORKSPACE;
  if (need > 0 && !aligned(workspace, 16)) return QMM_E_ALIGN;
  return QMM_OK;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct QmoeLayout {
  size_t h = 0, sync = 0, xq = 0, xs = 0, hq = 0, hs = 0, total = 0;
};

// The sync words sit at offset 0 for every shape and mode, so calls of different
// shapes on one buffer (the no-allocation entry's static array) never find another
// shape's h or codes where their sync words are.
QmoeLayout qmoe_layout(int64_t T, int64_t H, int64_t I, int k, int mode) {
  QmoeLayout L;
  size_t off = 0;
  L.sync = off;
  off += align256((size_t)kQmoeSyncWords * 4);
  L.h = off;
  off += align256((size_t)(T * k * I) * 2);
  if (mode == QMOE_INT8_ACT) {
    L.xq = off;
    off += align256((size_t)(T * H));
    L.xs = off;
    off += align256((size_t)(T * (H / 32)) * 4);
    L.hq = off;
    off += align256((size_t)(T * k * I));
    L.hs = off;
    off += align256((size_t)(T * k * (I / 32)) * 4);
  }
  L.total = off;
  return L;
}

constexpr size_t kMaxLds = 64 * 1024;
constexpr size_t kMaxFpLds = 160 * 1024;

qmm_status check_qmoe(const uint16_t* X, int64_t T, int64_t H, int64_t I, int64_t E, int k,
                      const int32_t* ids, const float* w, qmoe_weights fc1, qmoe_weights fc2,
                      int bits, int block, int mode, const uint16_t* Y, const void* scratch,
                      size_t scratch_bytes) {
  if (bits != 4) return QMM_E_BITS;
  if (!is_pow2_block(block) || block < 32) return QMM_E_BLOCK;
  if (mode != QMOE_FP && mode != QMOE_INT8_ACT) return QMM_E_MODE;
  if (T < 0 || T > 4096 || H <= 0 || I <= 0 || H > (1LL << 24) || I > (1LL << 24)) return QMM_E_SHAPE;
  if (E < 1 || E > (1LL << 20) || k < 1 || k > 64 || k > E) return QMM_E_SHAPE;
  if (H % 8 != 0 || I % 8 != 0) return QMM_E_SHAPE;
  if (mode == QMOE_INT8_ACT) {
    if (H % 32 != 0 || I % 32 != 0) return QMM_E_SHAPE;
    if ((size_t)H + (size_t)(H / 32) * 8 > kMaxLds) return QMM_E_SHAPE;
    if ((size_t)(k * I) + (size_t)(k * I / 32) * 8 > kMaxLds) return QMM_E_SHAPE;
  } else {
    // fp mode stages x (fc1) and the k rows of h (fc2) in LDS as fp32 plus chunk sums
    if ((size_t)ceil_div(H, 32) * 33 * 4 > kMaxFpLds) return QMM_E_SHAPE;
    if ((size_t)k * (size_t)ceil_div(I, 32) * 33 * 4 > kMaxFpLds) return QMM_E_SHAPE;
  }
  if (T == 0) return QMM_OK;
  if (!X || !ids || !w || !Y) return QMM_E_NULL;
  if (!fc1.W || !fc1.scales || !fc2.W || !fc2.scales) return QMM_E_NULL;
  if (!aligned(X, 16) || !aligned(Y, 2) || !aligned(ids, 4) || !aligned(w, 4)) return QMM_E_ALIGN;
  if (!aligned(fc1.W, 16) || !aligned(fc2.W, 16) || !aligned(fc1.scales, 2) ||
      !aligned(fc2.scales, 2) || !aligned(fc1.bias, 2) || !aligned(fc2.bias, 2))
    return QMM_E_ALIGN;
  const size_t need = qmoe_layout(T, H, I, k, mode).total;
  if (!scratch || scratch_bytes < need) return QMM_E_WORKSPACE;
  if (!aligned(scratch, 256)) return QMM_E_ALIGN;
  return QMM_OK;
}

GemvArgs make_gemv(const void* A, int a_type, int64_t M, int64_t K, int64_t N, const uint8_t* W,
                   int bits, int block, const void* bias, void* C, int c_type) {
  GemvArgs g{};
  g.A = A;
  g.a_type = a_type;
  g.M = M;
  g.K = K;
  g.N = N;
  g.W = W;
  g.bits = bits;
  g.block = block;
  g.block_log2 = __builtin_ctz((unsigned)block);
  g.nblk = ceil_div(K, block);
  g.row_bytes = g.nblk * block * bits / 8;
  const int64_t chb = bits == 3 ? 12 : 16;  // bytes of a lane's weight chunk (32 3-bit codes)
  g.nchunks = g.row_bytes / chb;
  g.bias = bias;
  g.C = C;
  g.c_type = c_type;
  g.chunked = (g.row_bytes % chb == 0) && aligned(W, 16);
  g.lpr_log2 = gemv_row_lanes_log2(g.nchunks, N);
  g.a_vec = aligned(A, 16) && (K % 4 == 0);
  return g;
}

// Run a GEMV over all M rows, at most kMaxGemvM rows of A per launch.
hipError_t run_gemv_rows(int entry, GemvArgs g, hipStream_t st) {
  const size_t a_es = dtype_size(g.a_type), c_es = dtype_size(g.c_type);
  for (int64_t m0 = 0; m0 < g.M; m0 += kMaxGemvM) {
    GemvArgs s = g;
    s.M = std::min<int64_t>(kMaxGemvM, g.M - m0);
    s.A = (const uint8_t*)g.A + m0 * g.K * (int64_t)a_es;
    s.C = (uint8_t*)g.C + m0 * g.N * (int64_t)c_es;
    s.a_vec = g.a_vec && aligned(s.A, 16);
    gemv_plan(s, device_cus());
    const int R = gemv_choice(entry, s, st);
    hipError_t e = launch_gemv(s, R, st);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

// ===========================================================================
// extern "C" entry points
// ===========================================================================
extern "C" {

size_t qmm_nbits_workspace_bytes(int64_t M, int64_t K, int64_t N, int a_type) {
  // the prefill path (M > 8) writes A once as fp16 rows of K rounded up to 64
  // (zero padded) into the workspace, whatever the type of A; when the output tiles
  // do not fill the chip the reduction is split and fp32 partial sums follow A
  (void)a_type;
  if (M <= kMaxGemvM || M <= 0 || K <= 0 || N <= 0) return 0;
  return matrix_workspace_bytes(M, K, N);
}

size_t qmm_codebook4_workspace_bytes(int64_t M, int64_t K, int64_t N, int a_type) {
  // the matrix-core paths take the workspace of qmm_nbits: M > 8, and 4 <= M <= 8 with
  // a 16-bit output (the output type is not an argument, so the size covers that case)
  // except M = 4 on a shape the GEMV keeps
  (void)a_type;
  if (M < kCbSkinnyMinM || K <= 0 || N <= 0 || codebook_gemv_m4(M, K, N)) return 0;
  return matrix_workspace_bytes(M, K, N);
}

qmm_status qmm_validate_nbits(const void* A, int a_type, int64_t M, int64_t K, int64_t N,
                              const uint8_t* W, int bits, int block, const uint16_t* scales,
                              const void* zp, int zp_kind, const void* bias, const void* C,
                              int c_type, const void* workspace, size_t workspace_bytes) {
  return check_nbits(A, a_type, M, K, N, W, bits, block, scales, zp, zp_kind, bias, C, c_type,
                     workspace, workspace_bytes);
}

qmm_status qmm_validate_codebook4(const void* A, int a_type, int64_t M, int64_t K, int64_t N,
                                  const uint8_t* W, int block, const float* absmax,
                                  const float* codebook, const void* bias, const void* C,
                                  int c_type, const void* workspace, size_t workspace_bytes) {
  return check_codebook(A, a_type, M, K, N, W, block, absmax, codebook, bias, C, c_type,
                        workspace, workspace_bytes);
}

qmm_status qmm_nbits(const void* A, int a_type, int64_t M, int64_t K, int64_t N, const uint8_t* W,
                     int bits, int block, const uint16_t* scales, const void* zp, int zp_kind,
                     float uniform_zp, const void* bias, void* C, int c_type, void* workspace,
                     size_t workspace_bytes, void* stream) {
  (void)hipGetLastError();
  const qmm_status s = check_nbits(A, a_type, M, K, N, W, bits, block, scales, zp, zp_kind, bias, C,
                                   c_type, workspace, workspace_bytes);
  if (s != QMM_OK) return s;
  if (M == 0 || N == 0) return QMM_OK;
  hipStream_t st = (hipStream_t)stream;
  if (M > kMaxGemvM && K > 0) {
    // prefill: A -> fp16 once (or fp16 A in place), then a matrix-core kernel
    PrefillArgs p{};
    const int64_t Kp = (K + 63) / 64 * 64;
    p.M = M;
    p.N = N;
    p.K = K;
    p.Kp = Kp;
    p.ldc = N;
    p.W = W;
    p.bits = bits;
    p.block = block;
    p.block_log2 = __builtin_ctz((unsigned)block);
    p.nblk = ceil_div(K, block);
    p.row_bytes = p.nblk * block * bits / 8;
    p.scales = scales;
    p.zp = zp;
    p.zp_kind = zp_kind;
    p.zconst = zp_kind == QMM_ZP_UNIFORM ? uniform_zp : default_zp(bits);
    p.zconst_fma = zconst_fma_exact(p.zconst) ? 1 : 0;
    p.zp_row_bytes = ceil_div(p.nblk * bits, 8);
    p.bias = bias;
    p.C = C;
    p.c_type = c_type;
    // a few rows: the skinny kernel (16-row tiles, each weight dequantized once)
    const bool skinny = skinny_applies(M, N, Kp, block, p.row_bytes, p.nblk);
    hipError_t e = matrix_activations(p, A, a_type, skinny, workspace, st);
    if (e == hipSuccess) e = skinny ? launch_skinny(p, st) : launch_prefill(p, st);
    if (e != hipSuccess) return (qmm_status)e;
    return (qmm_status)hipGetLastError();
  }
  GemvArgs g = make_gemv(A, a_type, M, K, N, W, bits, block, bias, C, c_type);
  g.fmt = GEMV_AFFINE;
  g.scales = scales;
  g.zp = zp;
  g.zp_kind = zp_kind;
  g.uniform_zp = uniform_zp;
  g.zp_row_bytes = ceil_div(g.nblk * bits, 8);
  hipError_t e = run_gemv_rows(ENTRY_NBITS, g, st);
  if (e != hipSuccess) return (qmm_status)e;
  return (qmm_status)hipGetLastError();
}

qmm_status qmm_codebook4(const void* A, int a_type, int64_t M, int64_t K, int64_t N,
                         const uint8_t* W, int block, const float* absmax, const float* codebook,
                         const void* bias, void* C, int c_type, void* workspace,
                         size_t workspace_bytes, void* stream) {
  (void)hipGetLastError();
  const qmm_status s = check_codebook(A, a_type, M, K, N, W, block, absmax, codebook, bias, C,
                                      c_type, workspace, workspace_bytes);
  if (s != QMM_OK) return s;
  if (M == 0 || N == 0) return QMM_OK;
  hipStream_t st = (hipStream_t)stream;
  if (codebook_on_matrix_cores(M, K, N, block, c_type)) {
    // matrix-core path: A -> padded fp16 once (or fp16 A in place),
    // W16 = fp16(codebook[q] * absmax) per tile
    PrefillArgs p{};
    const int64_t Kp = (K + 63) / 64 * 64;
    p.M = M;
    p.N = N;
    p.K = K;
    p.Kp = Kp;
    p.ldc = N;
    p.W = W;
    p.bits = 4;
    p.block = block;
    p.block_log2 = __builtin_ctz((unsigned)block);
    p.nblk = ceil_div(K, block);
    p.row_bytes = p.nblk * block / 2;
    p.fmt = GEMV_CODEBOOK;
    p.absmax = absmax;
    p.codebook = codebook;
    p.zp_kind = QMM_ZP_NONE;
    p.bias = bias;
    p.C = C;
    p.c_type = c_type;
    // a few rows: the skinny kernel (16-row tiles, each weight dequantized once)
    const bool skinny = skinny_applies(M, N, Kp, block, p.row_bytes, p.nblk);
    hipError_t e = matrix_activations(p, A, a_type, skinny, workspace, st);
    if (e == hipSuccess) e = skinny ? launch_skinny(p, st) : launch_prefill(p, st);
    if (e != hipSuccess) return (qmm_status)e;
    return (qmm_status)hipGetLastError();
  }
  GemvArgs g = make_gemv(A, a_type, M, K, N, W, 4, block, bias, C, c_type);
  g.fmt = GEMV_CODEBOOK;
  g.absmax = absmax;
  g.codebook = codebook;
  hipError_t e = run_gemv_rows(ENTRY_CODEBOOK, g, st);
  if (e != hipSuccess) return (qmm_status)e;
  return (qmm_status)hipGetLastError();
}

static qmm_status check_nested(const qmm_nested_absmax* a) {
  if (!a) return QMM_E_NULL;
  if (a->group < 1) return QMM_E_SHAPE;
  if (!a->codes || !a->table || !a->scales) return QMM_E_NULL;
  if (!aligned(a->table, 4) || !aligned(a->scales, 4)) return QMM_E_ALIGN;
  return QMM_OK;
}

qmm_status qmm_dequantize_absmax_nested(const qmm_nested_absmax* absmax, int64_t count, float* out, void* stream) {
  (void)hipGetLastError();
  if (count < 0) return QMM_E_SHAPE;
  if (count == 0) return QMM_OK;
  const qmm_status s = check_nested(absmax);
  if (s != QMM_OK) return s;
  if (!out) return QMM_E_NULL;
  if (!aligned(out, 4)) return QMM_E_ALIGN;
  const hipError_t e = launch_nested_absmax(absmax->codes, absmax->table, absmax->scales, absmax->offset,
                                            absmax->group, count, out, (hipStream_t)stream);
  if (e != hipSuccess) return (qmm_status)e;
  return (qmm_status)hipGetLastError();
}

size_t qmm_codebook4_nested_workspace_bytes(int64_t M, int64_t K, int64_t N, int a_type, int block) {
  if (M <= 0 || K <= 0 || N <= 0 || !is_pow2_block(block)) return 0;
  const size_t am = ((size_t)N * (size_t)ceil_div(K, block) * 4 + 255) & ~size_t(255);
  return am + qmm_codebook4_workspace_bytes(M, K, N, a_type);
}

qmm_status qmm_codebook4_nested(const void* A, int a_type, int64_t M, int64_t K, int64_t N, const uint8_t* W,
                                int block, const qmm_nested_absmax* absmax, const float* codebook,
                                const void* bias, void* C, int c_type, void* workspace, size_t workspace_bytes,
                                void* stream) {
  (void)hipGetLastError();
  if (!is_pow2_block(block)) return QMM_E_BLOCK;
  if (M < 0 || K < 0 || N < 0 || M > (1LL << 30) || K > (1LL << 30) || N > (1LL << 30)) return QMM_E_SHAPE;
  if (M == 0 || N == 0) return QMM_OK;
  qmm_status s = K > 0 ? check_nested(absmax) : QMM_OK;
  if (s != QMM_OK) return s;
  const size_t need = qmm_codebook4_nested_workspace_bytes(M, K, N, a_type, block);
  if (need > 0 && (!workspace || workspace_bytes < need)) return QMM_E_WORKSPACE;
  if (need > 0 && !aligned(workspace, 256)) return QMM_E_ALIGN;
  const size_t am_bytes = K > 0 ? (((size_t)N * (size_t)ceil_div(K, block) * 4 + 255) & ~size_t(255)) : 0;
  float* am = (float*)workspace;
  // the regular entry's own checks, with the decoded absmax in place of a caller's
  s = check_codebook(A, a_type, M, K, N, W, block, K > 0 ? am : nullptr, codebook, bias, C, c_type,
                     (uint8_t*)workspace + am_bytes, workspace_bytes - am_bytes);
  if (s != QMM_OK) return s;
  if (K > 0) {
    const hipError_t e = launch_nested_absmax(absmax->codes, absmax->table, absmax->scales, absmax->offset,
                                              absmax->group, N * ceil_div(K, block), am, (hipStream_t)stream);
    if (e != hipSuccess) return (qmm_status)e;
    const hipError_t le = hipGetLastError();
    if (le != hipSuccess) return (qmm_status)le;
  }
  return qmm_codebook4(A, a_type, M, K, N, W, block, am, codebook, bias, C, c_type, (uint8_t*)workspace + am_bytes,
                       workspace_bytes - am_bytes, stream);
}

size_t qmm_uniform_scratch_bytes(void) { return (2 + kUniformPartials) * sizeof(uint32_t); }

qmm_status qmm_fp16_uniform_value(const uint16_t* zp, int64_t count, void* scratch,
                                  size_t scratch_bytes, int* is_uniform, float* value,
                                  void* stream) {
  (void)hipGetLastError();
  if (!is_uniform || !value) return QMM_E_NULL;
  *is_uniform = 0;
  *value = 0.0f;
  if (count < 0) return QMM_E_SHAPE;
  if (count == 0) return QMM_OK;
  if (!zp || !scratch) return QMM_E_NULL;
  if (scratch_bytes < qmm_uniform_scratch_bytes()) return QMM_E_WORKSPACE;
  if (!aligned(zp, 2) || !aligned(scratch, 4)) return QMM_E_ALIGN;
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = launch_uniform_check(zp, count, (uint32_t*)scratch, st);
  if (e != hipSuccess) return (qmm_status)e;
  uint32_t res[2] = {0, 0};
  e = hipMemcpyAsync(res, scratch, sizeof(res), hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return (qmm_status)e;
  *is_uniform = res[0] ? 1 : 0;
  std::memcpy(value, &res[1], 4);
  return (qmm_status)hipGetLastError();
}

qmm_status qmm_dequantize_nbits(const uint8_t* W, int bits, int block, const uint16_t* scales,
                                const void* zp, int zp_kind, float uniform_zp, int64_t N, int64_t K,
                                void* out, int out_type, void* stream) {
  (void)hipGetLastError();
  if (bits != 2 && bits != 3 && bits != 4 && bits != 8) return QMM_E_BITS;
  if (!is_pow2_block(block) || (bits == 3 && block < 32)) return QMM_E_BLOCK;
  if (N < 0 || K < 0) return QMM_E_SHAPE;
  if (out_type != QMM_F32 && out_type != QMM_F16) return QMM_E_DTYPE;
  if (zp_kind < QMM_ZP_NONE || zp_kind > QMM_ZP_UNIFORM) return QMM_E_MODE;
  if (N == 0 || K == 0) return QMM_OK;
  if (!W || !scales || !out) return QMM_E_NULL;
  if ((zp_kind == QMM_ZP_PACKED || zp_kind == QMM_ZP_F16) && !zp) return QMM_E_NULL;
  DequantArgs d{};
  d.W = W;
  d.fmt = GEMV_AFFINE;
  d.bits = bits;
  d.block = block;
  d.N = N;
  d.K = K;
  d.nblk = ceil_div(K, block);
  d.row_bytes = d.nblk * block * bits / 8;
  d.scales = scales;
  d.zp = zp;
  d.zp_kind = zp_kind;
  d.uniform_zp = uniform_zp;
  d.zp_row_bytes = ceil_div(d.nblk * bits, 8);
  d.out = out;
  d.out_type = out_type;
  const hipError_t e = launch_dequant(d, (hipStream_t)stream);
  if (e != hipSuccess) return (qmm_status)e;
  return (qmm_status)hipGetLastError();
}

qmm_status qmm_dequantize_codebook4(const uint8_t* W, int block, const float* absmax,
                                    const float* codebook, int64_t N, int64_t K, void* out,
                                    int out_type, void* stream) {
  (void)hipGetLastError();
  if (!is_pow2_block(block)) return QMM_E_BLOCK;
  if (N < 0 || K < 0) return QMM_E_SHAPE;
  if (out_type != QMM_F32 && out_type != QMM_F16) return QMM_E_DTYPE;
  if (N == 0 || K == 0) return QMM_OK;
  if (!W || !absmax || !codebook || !out) return QMM_E_NULL;
  DequantArgs d{};
  d.W = W;
  d.fmt = GEMV_CODEBOOK;
  d.bits = 4;
  d.block = block;
  d.N = N;
  d.K = K;
  d.nblk = ceil_div(K, block);
  d.row_bytes = d.nblk * block / 2;
  d.absmax = absmax;
  d.codebook = codebook;
  d.out = out;
  d.out_type = out_type;
  const hipError_t e = launch_dequant(d, (hipStream_t)stream);
  if (e != hipSuccess) return (qmm_status)e;
  return (qmm_status)hipGetLastError();
}

size_t qmoe_decode_scratch_bytes(int64_t T, int64_t H, int64_t I, int k, int mode) {
  if (T < 0 || H < 0 || I < 0 || k < 0) return 0;
  return qmoe_layout(T, H, I, k, mode).total;
}

qmm_status qmm_validate_qmoe(const uint16_t* X, int64_t T, int64_t H, int64_t I, int64_t E, int k,
                             const int32_t* expert_ids, const float* expert_w, qmoe_weights fc1,
                             qmoe_weights fc2, int bits, int block, int mode, const uint16_t* Y,
                             const void* scratch, size_t scratch_bytes) {
  return check_qmoe(X, T, H, I, E, k, expert_ids, expert_w, fc1, fc2, bits, block, mode, Y, scratch,
                    scratch_bytes);
}

qmm_status qmoe_decode_fused(const uint16_t* X, int64_t T, int64_t H, int64_t I, int64_t E, int k,
                             const int32_t* expert_ids, const float* expert_w, qmoe_weights fc1,
                             qmoe_weights fc2, int bits, int block, int mode, uint16_t* Y,
                             void* scratch, size_t scratch_bytes, void* stream) {
  (void)hipGetLastError();
  return qmm::qmoe_decode_run(X, T, H, I, E, k, expert_ids, expert_w, fc1, fc2, bits, block, mode, Y, scratch,
                              scratch_bytes, stream, true);
}

}  // extern "C"

// The MoE decode behind both entry points: may_time = false never times candidates
// (the cached choice of the shape or the default tiling), so the call allocates nothing.
qmm_status qmm::qmoe_decode_run(const uint16_t* X, int64_t T, int64_t H, int64_t I, int64_t E, int k,
                                const int32_t* expert_ids, const float* expert_w, qmoe_weights fc1,
                                qmoe_weights fc2, int bits, int block, int mode, uint16_t* Y, void* scratch,
                                size_t scratch_bytes, void* stream, bool may_time) {
  const qmm_status s = check_qmoe(X, T, H, I, E, k, expert_ids, expert_w, fc1, fc2, bits, block,
                                  mode, Y, scratch, scratch_bytes);
  if (s != QMM_OK) return s;
  if (T == 0) return QMM_OK;
  hipStream_t st = (hipStream_t)stream;
  QmoeArgs a{};
  a.X = X;
  a.T = T;
  a.H = H;
  a.I = I;
  a.E = E;
  a.k = k;
  a.ids = expert_ids;
  a.rw = expert_w;
  a.fc1 = fc1;
  a.fc2 = fc2;
  a.block = block;
  a.mode = mode;
  a.fc1_nblk = ceil_div(H, block);
  a.fc1_row_bytes = a.fc1_nblk * block / 2;
  a.fc1_zp_row_bytes = ceil_div(a.fc1_nblk, 2);
  a.fc1_chunks = ceil_div(H, 32);
  a.fc1_lpr_log2 = gemv_lanes_per_row_log2(a.fc1_chunks);
  a.fc2_nblk = ceil_div(I, block);
  a.fc2_row_bytes = a.fc2_nblk * block / 2;
  a.fc2_zp_row_bytes = ceil_div(a.fc2_nblk, 2);
  a.fc2_chunks = ceil_div(I, 32);
  a.fc2_lpr_log2 = gemv_lanes_per_row_log2(a.fc2_chunks);
  a.num_cus = device_cus();
  const QmoeLayout L = qmoe_layout(T, H, I, k, mode);
  uint8_t* sc = (uint8_t*)scratch;
  a.h = (uint16_t*)(sc + L.h);
  if (mode == QMOE_INT8_ACT) {
    a.xq_out = (int8_t*)(sc + L.xq);
    a.xs_out = (float*)(sc + L.xs);
    a.hq_out = (int8_t*)(sc + L.hq);
    a.hs_out = (float*)(sc + L.hs);
  }
  a.Y = Y;
  a.sync = (uint32_t*)(sc + L.sync);
  int r1 = 1, r2 = 1;
  qmoe_choice(a, st, may_time, &r1, &r2);
  if (qmoe_fused_choice(a, st, may_time, r1, r2) >= 0) {
    const hipError_t e = launch_qmoe_fused(a, st);  // the plan has checked that it fits
    if (e != hipSuccess) return (qmm_status)e;
    return (qmm_status)hipGetLastError();
  }
  hipError_t e = launch_qmoe_fc1(a, r1, st);
  if (e == hipSuccess) e = launch_qmoe_fc2(a, r2, st);
  if (e != hipSuccess) return (qmm_status)e;
  return (qmm_status)hipGetLastError();
}

extern "C" {

qmm_status qmoe_ragged_mm(const uint16_t* X, int64_t R, int64_t K, int64_t N, int64_t E,
                          const int32_t* row_offsets, qmoe_weights w, int bits, int block, uint16_t* Y,
                          void* stream) {
  (void)hipGetLastError();
  if (bits != 4) return QMM_E_BITS;
  if (!is_pow2_block(block) || block < 32) return QMM_E_BLOCK;
  if (R < 0 || K <= 0 || N <= 0 || E < 1 || E > (1LL << 20) || K % 8 != 0) return QMM_E_SHAPE;
  const int64_t nblk = ceil_div(K, block);
  const int64_t row_bytes = nblk * block / 2;
  // 32-bit buffer offsets: X, and one expert's weights and scales
  if (R * K * 2 >= (1LL << 31) || N * row_bytes >= (1LL << 31) || N * nblk * 2 >= (1LL << 31) ||
      R >= (1LL << 31) - 64)
    return QMM_E_SHAPE;
  if (R == 0) return QMM_OK;
  if (!X || !row_offsets || !w.W || !w.scales || !Y) return QMM_E_NULL;
  if (!aligned(X, 16) || !aligned(Y, 2) || !aligned(row_offsets, 4) || !aligned(w.W, 16) ||
      !aligned(w.scales, 2) || !aligned(w.bias, 2))
    return QMM_E_ALIGN;
  RaggedArgs p{};
  p.X = X;
  p.R = R;
  p.K = K;
  p.N = N;
  p.E = E;
  p.offsets = row_offsets;
  p.W = w.W;
  p.scales = w.scales;
  p.zp = w.zp;
  p.bias = w.bias;
  p.block = block;
  p.block_log2 = __builtin_ctz((unsigned)block);
  p.nblk = nblk;
  p.row_bytes = row_bytes;
  p.zp_row_bytes = ceil_div(nblk, 2);
  p.Y = Y;
  const hipError_t e = launch_ragged(p, (hipStream_t)stream);
  if (e != hipSuccess) return (qmm_status)e;
  return (qmm_status)hipGetLastError();
}

qmm_status qmoe_decode_status(void* scratch, size_t scratch_bytes, int64_t T, int64_t H, int64_t I, int k,
                              int mode, int* timed_out, void* stream) {
  (void)hipGetLastError();
  if (!timed_out) return QMM_E_NULL;
  *timed_out = 0;
  if (mode != QMOE_FP && mode != QMOE_INT8_ACT) return QMM_E_MODE;
  if (T < 0 || H < 0 || I < 0 || k < 0) return QMM_E_SHAPE;
  if (T == 0) return QMM_OK;
  const QmoeLayout L = qmoe_layout(T, H, I, k, mode);
  if (!scratch) return QMM_E_NULL;
  if (scratch_bytes < L.total) return QMM_E_WORKSPACE;
  if (!aligned(scratch, 256)) return QMM_E_ALIGN;
  hipStream_t st = (hipStream_t)stream;
  uint32_t* flag = (uint32_t*)((uint8_t*)scratch + L.sync) + 2;
  uint32_t v = 0;
  hipError_t e = hipMemcpyAsync(&v, flag, 4, hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e == hipSuccess && v != 0) {
    e = hipMemsetAsync(flag, 0, 4, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
  }
  if (e != hipSuccess) return (qmm_status)e;
  *timed_out = v != 0 ? 1 : 0;
  return QMM_OK;
}

// ---- activation quantization ops ---------------------------------------------
static qmm_status check_qparams(qmm_qparams q, int bits) {
  if (!(q.scale > 0.0f) || !(q.scale <= 3.402823466e38f)) return QMM_E_PARAM;
  if (q.zero_point < 0 || q.zero_point > (1 << bits) - 1) return QMM_E_PARAM;
  return QMM_OK;
}

static qmm_status check_qdq_common(int64_t n, int bits) {
  if (bits != 8 && bits != 16) return QMM_E_BITS;
  if (n < 0) return QMM_E_SHAPE;
  return QMM_OK;
}

static bool codes_aligned(const void* p, int bits) { return aligned(p, bits == 16 ? 2 : 1); }

qmm_status qmm_quantize_linear(const void* x, int x_type, int64_t n, qmm_qparams q, int bits, void* codes,
                               void* stream) {
  (void)hipGetLastError();
  qmm_status s = check_qdq_common(n, bits);
  if (s != QMM_OK) return s;
  if (!valid_dtype(x_type)) return QMM_E_DTYPE;
  if ((s = check_qparams(q, bits)) != QMM_OK) return s;
  if (n == 0) return QMM_OK;
  if (!x || !codes) return QMM_E_NULL;
  if (!aligned(x, dtype_size(x_type)) || !codes_aligned(codes, bits)) return QMM_E_ALIGN;
  const hipError_t e = launch_quantize_linear(x, x_type, n, q, bits, codes, (hipStream_t)stream);
  if (e != hipSuccess) return (qmm_status)e;
  return (qmm_status)hipGetLastError();
}

qmm_status qmm_dequantize_linear(const void* codes, int64_t n, qmm_qparams q, int bits, void* y, int y_type,
                                 void* stream) {
  (void)hipGetLastError();
  qmm_status s = check_qdq_common(n, bits);
  if (s != QMM_OK) return s;
  if (!valid_dtype(y_type)) return QMM_E_DTYPE;
  if ((s = check_qparams(q, bits)) != QMM_OK) return s;
  if (n == 0) return QMM_OK;
  if (!codes || !y) return QMM_E_NULL;
  if (!aligned(y, dtype_size(y_type)) || !codes_aligned(codes, bits)) return QMM_E_ALIGN;
  const hipError_t e = launch_dequantize_linear(codes, n, q, bits, y, y_type, (hipStream_t)stream);
  if (e != hipSuccess) return (qmm_status)e;
  return (qmm_status)hipGetLastError();
}

qmm_status qmm_fake_quantize(const void* x, int x_type, int64_t n, qmm_qparams q, int bits, void* y,
                             void* stream) {
  (void)hipGetLastError();
  qmm_status s = check_qdq_common(n, bits);
  if (s != QMM_OK) return s;
  if (!valid_dtype(x_type)) return QMM_E_DTYPE;
  if ((s = check_qparams(q, bits)) != QMM_OK) return s;
  if (n == 0) return QMM_OK;
  if (!x || !y) return QMM_E_NULL;
  if (!aligned(x, dtype_size(x_type)) || !aligned(y, dtype_size(x_type))) return QMM_E_ALIGN;
  const hipError_t e = launch_fake_quantize(x, x_type, n, q, bits, y, (hipStream_t)stream);
  if (e != hipSuccess) return (qmm_status)e;
  return (qmm_status)hipGetLastError();
}

qmm_status qmm_qsigmoid(const void* codes_in, int64_t n, qmm_qparams in, qmm_qparams out, int bits,
                        void* codes_out, void* stream) {
  (void)hipGetLastError();
  qmm_status s = check_qdq_common(n, bits);
  if (s != QMM_OK) return s;
  if ((s = check_qparams(in, bits)) != QMM_OK || (s = check_qparams(out, bits)) != QMM_OK) return s;
  if (n == 0) return QMM_OK;
  if (!codes_in || !codes_out) return QMM_E_NULL;
  if (!codes_aligned(codes_in, bits) || !codes_aligned(codes_out, bits)) return QMM_E_ALIGN;
  const hipError_t e = launch_qsigmoid(codes_in, n, in, out, bits, codes_out, (hipStream_t)stream);
  if (e != hipSuccess) return (qmm_status)e;
  return (qmm_status)hipGetLastError();
}

qmm_status qmm_qmul(const void* a, qmm_qparams qa, const void* b, qmm_qparams qb, int64_t n, qmm_qparams qc,
                    int bits, void* c, void* stream) {
  (void)hipGetLastError();
  qmm_status s = check_qdq_common(n, bits);
  if (s != QMM_OK) return s;
  if ((s = check_qparams(qa, bits)) != QMM_OK || (s = check_qparams(qb, bits)) != QMM_OK ||
      (s = check_qparams(qc, bits)) != QMM_OK)
    return s;
  if (n == 0) return QMM_OK;
  if (!a || !b || !c) return QMM_E_NULL;
  if (!codes_aligned(a, bits) || !codes_aligned(b, bits) || !codes_aligned(c, bits)) return QMM_E_ALIGN;
  const hipError_t e = launch_qmul(a, qa, b, qb, n, qc, bits, c, (hipStream_t)stream);
  if (e != hipSuccess) return (qmm_status)e;
  return (qmm_status)hipGetLastError();
}

qmm_status qmm_qswiglu(const void* gate, const void* up, int x_type, int64_t n, int bits, const qmm_qparams* q,
                       void* y, void* stream) {
  (void)hipGetLastError();
  qmm_status s = check_qdq_common(n, bits);
  if (s != QMM_OK) return s;
  if (!valid_dtype(x_type)) return QMM_E_DTYPE;
  if (!q) return QMM_E_NULL;
  for (int i = 0; i < 5; ++i)
    if ((s = check_qparams(q[i], bits)) != QMM_OK) return s;
  if (n == 0) return QMM_OK;
  if (!gate || !up || !y) return QMM_E_NULL;
  const size_t es = dtype_size(x_type);
  if (!aligned(gate, es) || !aligned(up, es) || !aligned(y, es)) return QMM_E_ALIGN;
  const hipError_t e = launch_qswiglu(gate, up, x_type, n, bits, q, y, (hipStream_t)stream);
  if (e != hipSuccess) return (qmm_status)e;
  return (qmm_status)hipGetLastError();
}

qmm_status qmm_set_tuning(int mode, int forced_index) {
  if (mode < 0 || mode > 2) return QMM_E_MODE;
  TunerState& t = tuner();
  std::lock_guard<std::mutex> lock(t.mu);
  t.mode = mode;
  t.forced = forced_index;
  return QMM_OK;
}

int qmm_nbits_gemv_matrix_core_form(int64_t M, int64_t K, int64_t N, int bits, int block) {
  if (M != 1 || K <= 0 || N <= 0 || bits != 2 || block < 16 || (block & (block - 1)) != 0) return 0;
  GemvArgs g = make_gemv((const void*)(uintptr_t)256, QMM_F32, M, K, N, (const uint8_t*)(uintptr_t)256, bits,
                         block, nullptr, nullptr, QMM_F32);
  gemv_plan(g, 256);
  return gemv_mx_supported(g) ? 1 : 0;
}

int qmm_num_candidates(int entry) {
  if (entry == ENTRY_NBITS || entry == ENTRY_CODEBOOK) return kNumGemvCandidates;
  if (entry == ENTRY_QMOE_FC1 || entry == ENTRY_QMOE_FC2) return kNumQmoeCandidates;
  if (entry == ENTRY_QMOE_FUSED) return kNumQmoeFused;
  return 0;
}

int qmm_tuned_choice(int entry) {
  if (entry < 0 || entry >= ENTRY_COUNT) return -1;
  TunerState& t = tuner();
  std::lock_guard<std::mutex> lock(t.mu);
  return t.last_choice[entry];
}

void qmm_clear_tuning(void) {
  TunerState& t = tuner();
  std::lock_guard<std::mutex> lock(t.mu);
  t.choice.clear();
  for (int i = 0; i < ENTRY_COUNT; ++i) t.last_choice[i] = -1;
}

int qmm_tuner_pick(const double* times_us, int rounds, int ncand) {
  if (!times_us || rounds < 2 || ncand < 1) return -1;
  return pick_winner(times_us, rounds, ncand);
}

int qmm_tuner_pick_single_launch(const double* times_us, int rounds, int ncand) {
  if (!times_us || rounds < 2 || ncand < 2) return -1;
  return pick_single_launch(times_us, rounds, ncand);
}

qmm_status qmm_hbm_read_probe(const void* buf, int64_t bytes, uint32_t* sink, int groups, void* stream) {
  (void)hipGetLastError();
  if (bytes < 0 || bytes % 16 != 0 || groups < 1 || groups > (1 << 20)) return QMM_E_SHAPE;
  if (bytes == 0) return QMM_OK;
  if (!buf || !sink) return QMM_E_NULL;
  if (!aligned(buf, 16) || !aligned(sink, 4)) return QMM_E_ALIGN;
  const hipError_t e = launch_hbm_read(buf, bytes, sink, groups, (hipStream_t)stream);
  if (e != hipSuccess) return (qmm_status)e;
  return (qmm_status)hipGetLastError();
}

qmm_status qmm_launch_timing_begin(int n) {
  LaunchTiming& t = g_launch_timing;
  if (t.on) return QMM_E_MODE;
  if (n < 1 || n > 65536) return QMM_E_SHAPE;
  t.start = new hipEvent_t[n];
  t.stop = new hipEvent_t[n];
  int made = 0;
  hipError_t e = hipSuccess;
  for (; made < n; ++made) {
    if ((e = hipEventCreate(&t.start[made])) != hipSuccess) break;
    if ((e = hipEventCreate(&t.stop[made])) != hipSuccess) {
      (void)hipEventDestroy(t.start[made]);
      break;
    }
  }
  if (e != hipSuccess) {
    for (int i = 0; i < made; ++i) {
      (void)hipEventDestroy(t.start[i]);
      (void)hipEventDestroy(t.stop[i]);
    }
    delete[] t.start;
    delete[] t.stop;
    t = LaunchTiming{};
    return (qmm_status)e;
  }
  t.cap = n;
  t.next = 0;
  t.on = 1;
  return QMM_OK;
}

qmm_status qmm_launch_timing_end(float* us, int n_max, int* count) {
  LaunchTiming& t = g_launch_timing;
  if (!count) return QMM_E_NULL;
  *count = 0;
  if (!t.on) return QMM_OK;
  hipError_t first = hipSuccess;
  const int used = t.next;
  for (int i = 0; i < used; ++i) {
    float ms = 0.0f;
    hipError_t e = hipEventSynchronize(t.stop[i]);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, t.start[i], t.stop[i]);
    if (e != hipSuccess && first == hipSuccess) first = e;
    if (us && i < n_max) us[i] = ms * 1000.0f;
  }
  for (int i = 0; i < t.cap; ++i) {
    (void)hipEventDestroy(t.start[i]);
    (void)hipEventDestroy(t.stop[i]);
  }
  delete[] t.start;
  delete[] t.stop;
  t = LaunchTiming{};
  *count = used;
  return (qmm_status)first;
}

const char* qmm_status_string(qmm_status s) {
  switch (s) {
    case QMM_OK: return "ok";
    case QMM_E_NULL: return "null pointer";
    case QMM_E_DTYPE: return "unsupported element type";
    case QMM_E_BITS: return "unsupported bit width";
    case QMM_E_BLOCK: return "unsupported block size";
    case QMM_E_SHAPE: return "bad shape";
    case QMM_E_ALIGN: return "misaligned pointer";
    case QMM_E_WORKSPACE: return "workspace missing or too small";
    case QMM_E_MODE: return "unknown mode or zero-point kind";
    case QMM_E_DEVICE: return "no usable device";
    case QMM_E_PARAM: return "quantization parameter out of range";
    default: return s > 0 ? hipGetErrorString((hipError_t)s) : "unknown status";
  }
}

}  // extern "C"
