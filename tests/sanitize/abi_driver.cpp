// Host driver for the sanitizer build of exact_io_aware_fa_amd/csrc/fa_api.cpp
// (AddressSanitizer and UndefinedBehaviorSanitizer).  The kernel launchers are
// replaced by stubs that count calls and record their arguments, so every
// validation path of every entry point runs on the CPU: each bad argument must
// return its status before any launch, each valid call must reach exactly one
// launcher with the workspace carved as documented.  No pointer passed here is
// dereferenced by the library.  Prints "ABI SANITIZE OK" and returns 0 when
// every check holds.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "fa.h"
#include "fa_kernels.h"

static int launches = 0;
static fa::DecodeArgs last_decode;
namespace fa {
hipError_t launch_prefill_bf16(const PrefillArgs&) { ++launches; return hipSuccess; }
hipError_t launch_prefill_f32(const PrefillArgs&) { ++launches; return hipSuccess; }
hipError_t launch_bwd_bf16(const BwdArgs&) { ++launches; return hipSuccess; }
hipError_t launch_decode_bf16(const DecodeArgs& a) { ++launches; last_decode = a; return hipSuccess; }
hipError_t launch_decode_paged_bf16(const DecodeArgs& a) { ++launches; last_decode = a; return hipSuccess; }
int decode_max_group() { return 16; }
hipError_t decode_scratch(void** ptr, size_t* bytes) {
  *ptr = reinterpret_cast<void*>((uintptr_t)0x7000000000ull);
  *bytes = FA_DECODE_SCRATCH_BYTES;
  return hipSuccess;
}
}  // namespace fa
extern "C" const char* hipGetErrorString(hipError_t) { return "stub"; }

static int failures = 0;
static void expect(int got, int want, const char* what) {
  if (got != want) {
    std::fprintf(stderr, "%s: status %d, expected %d (%s)\n", what, got, want, fa_last_error());
    ++failures;
  }
}
// distinct, aligned fake device addresses, 8 GiB apart (more than any buffer here)
static void* P(int i) { return reinterpret_cast<void*>((uintptr_t)(0x100000000ull + (uint64_t)i * 0x200000000ull)); }
static float* F(int i) { return static_cast<float*>(P(i)); }
static const int32_t* I(int i) { return static_cast<const int32_t*>(P(i)); }

int main() {
  expect(fa_abi_version(), FA_ABI_VERSION, "abi version");
  for (int s = 0; s < 6; ++s)
    if (!fa_status_str((fa_status_t)s) || !std::strlen(fa_status_str((fa_status_t)s))) ++failures;

  // ---- fa_fwd
  auto fwd = [](int dt, int B, int Hq, int Hkv, int N, int Nk, int d, float sc, void* o = P(4), float* l = F(5)) {
    return (int)fa_fwd((fa_dtype_t)dt, P(1), P(2), P(3), o, l, B, Hq, Hkv, N, Nk, d, 1, sc, nullptr);
  };
  int before = launches;
  expect(fwd(FA_BF16, 2, 8, 2, 100, 130, 128, 0.1f), FA_OK, "fwd valid bf16");
  expect(fwd(FA_F32, 1, 1, 1, 256, 256, 64, 0.125f), FA_OK, "fwd valid f32");
  if (launches != before + 2) ++failures;
  before = launches;
  expect(fwd(9, 1, 1, 1, 4, 4, 64, 0.1f), FA_ERR_INVALID_ARG, "fwd dtype");
  expect(fwd(FA_BF16, -1, 1, 1, 4, 4, 64, 0.1f), FA_ERR_INVALID_ARG, "fwd B<0");
  expect(fwd(FA_BF16, 1, 3, 2, 4, 4, 64, 0.1f), FA_ERR_INVALID_ARG, "fwd Hq%Hkv");
  expect(fwd(FA_BF16, 1, 1, 1, 4, 4, 96, 0.1f), FA_ERR_UNSUPPORTED, "fwd d=96");
  expect(fwd(FA_BF16, 1, 1, 1, 4, 4, 64, NAN), FA_ERR_INVALID_ARG, "fwd scale nan");
  expect(fwd(FA_BF16, 1, 1, 1, 4, 4, 64, -1.0f), FA_ERR_INVALID_ARG, "fwd scale<0");
  expect(fwd(FA_BF16, 1, 1, 1, 4, 4, 64, 0.1f, P(1)), FA_ERR_INVALID_ARG, "fwd o aliases q");
  expect(fwd(FA_BF16, 1, 1, 1, 4, 4, 64, 0.1f, (char*)P(4) + 8), FA_ERR_INVALID_ARG, "fwd misaligned o");
  expect(fwd(FA_BF16, 1, 64, 8, 1 << 20, 1 << 20, 128, 0.1f), FA_ERR_UNSUPPORTED, "fwd slice over 2 GiB");
  expect(fwd(FA_BF16, 0, 1, 1, 4, 4, 64, 0.1f), FA_OK, "fwd B=0 no-op");
  if (launches != before) ++failures;

  // ---- fa_fwd_varlen
  before = launches;
  expect((int)fa_fwd_varlen(FA_BF16, P(1), P(2), P(3), I(6), I(7), 300, 900, 1000, 3000, P(4), F(5), 4, 8, 2, 128, 1,
                            0.1f, nullptr), FA_OK, "varlen valid");
  expect((int)fa_fwd_varlen(FA_F32, P(1), P(2), P(3), I(6), I(7), 300, 900, 1000, 3000, P(4), F(5), 4, 8, 2, 128, 1,
                            0.1f, nullptr), FA_ERR_UNSUPPORTED, "varlen f32");
  expect((int)fa_fwd_varlen(FA_BF16, P(1), P(2), P(3), nullptr, I(7), 300, 900, 1000, 3000, P(4), F(5), 4, 8, 2, 128,
                            1, 0.1f, nullptr), FA_ERR_INVALID_ARG, "varlen null cu");
  expect((int)fa_fwd_varlen(FA_BF16, P(1), P(2), P(3), (const int32_t*)((char*)P(6) + 2), I(7), 300, 900, 1000, 3000,
                            P(4), F(5), 4, 8, 2, 128, 1, 0.1f, nullptr), FA_ERR_INVALID_ARG, "varlen misaligned cu");
  if (launches != before + 1) ++failures;

  // ---- fa_decode: the workspace is the partial outputs then their LSEs
  const int B = 32, Hq = 64, Hkv = 8, d = 128, L = 32768;
  const size_t ws = fa_decode_workspace_bytes(B, Hq, Hkv, d, L);
  if (ws == 0 || fa_decode_workspace_bytes(0, Hq, Hkv, d, L) != 0) ++failures;
  before = launches;
  expect((int)fa_decode(FA_BF16, P(1), P(2), P(3), I(6), L, P(4), F(5), B, Hq, Hkv, d, 0.1f, P(8), ws, nullptr),
         FA_OK, "decode valid");
  if (launches != before + 1 || (char*)last_decode.part_o != (char*)P(8) ||
      (char*)last_decode.part_lse <= (char*)P(8) || (char*)last_decode.part_lse >= (char*)P(8) + ws)
    ++failures;
  expect((int)fa_decode(FA_BF16, P(1), P(2), P(3), I(6), L, P(4), F(5), B, Hq, Hkv, d, 0.1f, P(8), ws - 1, nullptr),
         FA_ERR_WORKSPACE, "decode small workspace");
  expect((int)fa_decode(FA_BF16, P(1), P(2), P(3), I(6), L, P(4), F(5), B, 64, 2, d, 0.1f, P(8), ws, nullptr),
         FA_ERR_UNSUPPORTED, "decode group of 32");
  expect((int)fa_decode(FA_BF16, P(1), P(2), P(3), I(6), L, P(4), F(5), B, Hq, Hkv, d, 0.1f, P(4), ws, nullptr),
         FA_ERR_INVALID_ARG, "decode workspace aliases o");

  // ---- fa_decode_noalloc: the partial results go to the static array
  before = launches;
  expect((int)fa_decode_noalloc(FA_BF16, P(1), P(2), P(3), I(6), L, P(4), F(5), B, Hq, Hkv, d, 0.1f, nullptr), FA_OK,
         "noalloc valid");
  if (launches != before + 1 || (uintptr_t)last_decode.part_o != 0x7000000000ull) ++failures;
  expect((int)fa_decode_noalloc(FA_BF16, P(1), P(2), P(3), I(6), 1 << 22, P(4), F(5), 64, 64, 1, d, 0.1f, nullptr),
         FA_ERR_UNSUPPORTED, "noalloc group of 64");
  expect((int)fa_decode_noalloc(FA_BF16, P(1), P(2), P(3), I(6), 1 << 22, P(4), F(5), 1024, 16, 1, d, 0.1f, nullptr),
         FA_ERR_WORKSPACE, "noalloc beyond the static array");
  expect((int)fa_decode_noalloc(FA_BF16, P(1), P(2), P(3), I(6), L, P(1), F(5), B, Hq, Hkv, d, 0.1f, nullptr),
         FA_ERR_INVALID_ARG, "noalloc o aliases q");
  if (launches != before + 1) ++failures;

  // ---- fa_decode_paged
  const size_t pws = fa_decode_paged_workspace_bytes(B, Hq, Hkv, d, L);
  before = launches;
  expect((int)fa_decode_paged(FA_BF16, P(1), P(10), P(11), P(2), P(3), I(6), I(7), 16000, 64, 520, L, P(4), F(5), B,
                              Hq, Hkv, d, 0.1f, P(8), pws, nullptr), FA_OK, "paged valid");
  if (launches != before + 1 || last_decode.cu_tiles != (int32_t*)P(8)) ++failures;
  expect((int)fa_decode_paged(FA_BF16, P(1), P(10), nullptr, P(2), P(3), I(6), I(7), 16000, 64, 520, L, P(4), F(5),
                              B, Hq, Hkv, d, 0.1f, P(8), pws, nullptr), FA_ERR_INVALID_ARG, "paged k_new without v_new");
  expect((int)fa_decode_paged(FA_BF16, P(1), P(10), P(11), P(2), P(3), I(6), I(7), 16000, 48, 520, L, P(4), F(5), B,
                              Hq, Hkv, d, 0.1f, P(8), pws, nullptr), FA_ERR_INVALID_ARG, "paged block size 48");
  expect((int)fa_decode_paged(FA_BF16, P(1), P(10), P(11), P(2), P(3), I(6), I(7), 16000, 64, 100, L, P(4), F(5), B,
                              Hq, Hkv, d, 0.1f, P(8), pws, nullptr), FA_ERR_INVALID_ARG, "paged table too short");

  // ---- fa_bwd
  const size_t bws = fa_bwd_workspace_bytes(1, 64, 8192);
  before = launches;
  expect((int)fa_bwd(FA_BF16, P(1), P(2), P(3), P(4), F(5), P(10), P(11), P(12), P(13), 1, 64, 8, 8192, 8192, 128, 1,
                     0.1f, P(8), bws, nullptr), FA_OK, "bwd valid");
  expect((int)fa_bwd(FA_BF16, nullptr, P(2), P(3), nullptr, nullptr, nullptr, nullptr, P(12), P(13), 1, 64, 8, 0, 64,
                     128, 1, 0.1f, nullptr, 0, nullptr), FA_OK, "bwd N=0 with keys");
  if (launches != before + 2) ++failures;
  expect((int)fa_bwd(FA_BF16, P(1), P(2), P(3), P(4), F(5), P(10), P(1), P(12), P(13), 1, 64, 8, 8192, 8192, 128, 1,
                     0.1f, P(8), bws, nullptr), FA_ERR_INVALID_ARG, "bwd dq aliases q");
  expect((int)fa_bwd(FA_BF16, P(1), P(2), P(3), P(4), F(5), P(10), P(11), P(12), P(13), 1, 64, 8, 8192, 8192, 128, 1,
                     0.1f, P(8), bws / 2, nullptr), FA_ERR_WORKSPACE, "bwd small workspace");

  if (failures) {
    std::fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  std::printf("ABI SANITIZE OK\n");
  return 0;
}
