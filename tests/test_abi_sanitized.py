"""Host AddressSanitizer / UndefinedBehaviorSanitizer build of the C ABI's
argument validation (csrc/api.cpp), CPU only.

api.cpp is compiled with g++ and both sanitizers and linked against stub
launchers generated from csrc/w4_internal.h (each returns hipSuccess without
touching memory; the *_fits predicates answer true).  A small driver then
calls every entry point with valid, empty, extreme and invalid arguments.
Any out-of-bounds access, signed overflow or other undefined behaviour in the
validation aborts the driver; the expected status of each call is checked."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "dequant_gemm_quantize_amd", "csrc")
ROCM = "/opt/rocm"

pytestmark = pytest.mark.skipif(shutil.which("g++") is None or not os.path.exists(f"{ROCM}/include/hip"),
                                reason="needs g++ and the HIP headers")


def _stubs() -> str:
    src = open(os.path.join(CSRC, "w4_internal.h")).read()
    out = ['#include "w4_internal.h"', "namespace w4 {"]
    for ret, name, args in re.findall(r"^(hipError_t|bool|size_t)\s+(\w+)\(([^;]*?)\);", src, flags=re.M | re.S):
        if name == "gptq_group_ok":      # the one predicate the validation depends on
            body = "return g > 0 && g % 32 == 0 && (g <= 128 ? 128 % g == 0 : g % 128 == 0);"
        elif ret == "size_t":
            body = "return 0;"
        else:
            body = "return hipSuccess;" if ret == "hipError_t" else "return true;"
        out.append(f"{ret} {name}({args}) {{ {body} }}")
    out.append("}  // namespace w4")
    return "\n".join(out) + "\n"


DRIVER = r'''
#include <cstdint>
#include <cstdio>
#include "../../include/w4.h"

static int fails = 0;
static void expect(int got, int want, const char* what) {
  if (got != want) {
    std::printf("%s: status %d, expected %d (%s)\n", what, got, want, w4_last_error());
    ++fails;
  }
}

int main() {
  alignas(16) static unsigned char buf[4096];
  void* A = buf;
  void* U = buf + 4;
  uint8_t* P = buf;
  const int64_t BIG = INT64_MAX;
  // quantize + pack, all four quantizers
  expect(quantize_pack_int4(A, W4_BF16, 4, 256, 128, P, A, A, W4_F16, nullptr), W4_OK, "qp ok");
  expect(quantize_pack_int4_sym(A, W4_F32, 4, 256, 32, P, A, A, W4_F32, nullptr), W4_OK, "qp sym ok");
  expect(quantize_pack_int4(A, W4_BF16, 4, 100, 32, P, A, A, W4_F16, nullptr), W4_EINVAL, "qp k%g");
  expect(quantize_pack_int4(A, W4_BF16, BIG, 256, 128, P, A, A, W4_F16, nullptr), W4_EINVAL, "qp n huge");
  expect(quantize_pack_int4(A, W4_BF16, 4, BIG - (BIG % 128), 128, P, A, A, W4_F16, nullptr), W4_EINVAL, "qp k huge");
  expect(quantize_pack_int4(U, W4_BF16, 4, 256, 128, P, A, A, W4_F16, nullptr), W4_EINVAL, "qp misaligned");
  expect(quantize_pack_int4(A, W4_BF16, 0, 256, 128, nullptr, nullptr, nullptr, W4_F16, nullptr), W4_OK, "qp empty");
  expect(quantize_pack_int4(A, W4_BF16, 4, 256, -32, P, A, A, W4_F16, nullptr), W4_EINVAL, "qp g<0");
  expect(quantize_pack_int4_sym_percentile(A, W4_BF16, 4, 256, 128, 99.9, P, A, A, W4_F16, nullptr), W4_OK, "pct ok");
  expect(quantize_pack_int4_sym_percentile(A, W4_BF16, 4, 256, 128, 0.0 / 0.0, P, A, A, W4_F16, nullptr), W4_EINVAL, "pct nan");
  expect(quantize_pack_int4_sym_mse(A, W4_BF16, 4, 256, 128, 1000, P, A, A, W4_F16, nullptr), W4_OK, "mse ok");
  expect(quantize_pack_int4_sym_mse(A, W4_BF16, 4, 256, 128, -5, P, A, A, W4_F16, nullptr), W4_EINVAL, "mse n<0");
  // dequant, activations, products
  expect(dequant_int4(P, A, A, W4_F16, 4, 256, 128, A, W4_BF16, nullptr), W4_OK, "dq ok");
  expect(dequant_int4(P, A, A, W4_F16, BIG, BIG, 128, A, W4_BF16, nullptr), W4_EINVAL, "dq huge");
  expect(quantize_act_int8(A, W4_BF16, 3, 256, (int8_t*)A, (float*)A, nullptr), W4_OK, "act ok");
  expect(quantize_act_int8(A, W4_BF16, BIG, 256, (int8_t*)A, (float*)A, nullptr), W4_EINVAL, "act huge");
  expect(quantize_act_int8(A, W4_BF16, (1LL << 24) - 1, 8, (int8_t*)A, (float*)A, nullptr), W4_OK, "act m max");
  expect(quantize_act_int8(A, W4_BF16, 1LL << 24, 8, (int8_t*)A, (float*)A, nullptr), W4_EINVAL, "act m 2^24");
  for (int64_t m : {1, 3, 16, 64, 100, 2048})
    expect(w4a16_matmul(A, W4_BF16, m, 4096, P, A, A, W4_F16, 11008, 128, A, W4_BF16, nullptr), W4_OK, "w4a16 ok");
  expect(w4a16_matmul(A, W4_F32, 5, 256, P, A, A, W4_F32, 96, 32, A, W4_F32, nullptr), W4_OK, "w4a16 f32");
  expect(w4a16_matmul(A, W4_BF16, BIG, 4096, P, A, A, W4_F16, BIG, 128, A, W4_BF16, nullptr), W4_EINVAL, "w4a16 huge");
  expect(w4a16_matmul_ws(A, W4_BF16, 256, 11008, P, A, A, W4_F16, 4096, 128, A, W4_BF16, A, 4096, nullptr), W4_OK, "w4a16 ws ok");
  expect(w4a16_matmul_ws(A, W4_BF16, 256, 11008, P, A, A, W4_F16, 4096, 128, A, W4_BF16, nullptr, 0, nullptr), W4_OK, "w4a16 ws null");
  expect(w4a16_matmul_ws(A, W4_BF16, 256, 11008, P, A, A, W4_F16, 4096, 128, A, W4_BF16, U, 4096, nullptr), W4_EINVAL, "w4a16 ws misaligned");
  expect(w4a16_matmul_ws(A, W4_BF16, BIG, 4096, P, A, A, W4_F16, BIG, 128, A, W4_BF16, A, 4096, nullptr), W4_EINVAL, "w4a16 ws huge");
  expect(w4a16_matmul_noalloc(A, W4_BF16, 256, 11008, P, A, A, W4_F16, 4096, 128, A, W4_BF16, nullptr), W4_OK, "noalloc ok");
  expect(w4a16_matmul_noalloc(A, W4_BF16, 256, 11008, P, A, A, W4_F16, 4096, 128, nullptr, W4_BF16, nullptr), W4_EINVAL, "noalloc y null");
  expect(w4a16_matmul_noalloc(A, W4_BF16, BIG, 4096, P, A, A, W4_F16, BIG, 128, A, W4_BF16, nullptr), W4_EINVAL, "noalloc huge");
  expect(w4a16_matmul_noalloc(A, W4_BF16, 0, 4096, P, A, A, W4_F16, 64, 128, A, W4_BF16, nullptr), W4_OK, "noalloc empty");
  expect((int)w4a16_matmul_workspace_size(BIG, BIG, BIG, 128, W4_BF16), 0, "ws size huge");
  expect((int)w4a16_matmul_workspace_size(256, 11008, 4096, 100, W4_BF16), 0, "ws size bad g");
  expect((int)w4a16_matmul_workspace_size(-1, 11008, 4096, 128, W4_BF16), 0, "ws size m<0");
  for (int64_t m : {1, 4, 16, 17, 512})
    expect(w4a8_matmul((int8_t*)A, (float*)A, m, 8192, P, A, A, W4_F16, 28672, 128, A, W4_BF16, nullptr), W4_OK, "w4a8 ok");
  expect(w4a8_matmul((int8_t*)A, (float*)U, 1, 8192, P, A, A, W4_F16, 28672, 128, A, W4_BF16, nullptr), W4_OK, "w4a8 scale 4B");
  expect(w4a8_matmul_ws((int8_t*)A, (float*)A, 512, 8192, P, A, A, W4_F16, 3584, 128, A, W4_BF16, A, 4096, nullptr), W4_OK, "w4a8 ws ok");
  expect(w4a8_matmul_ws((int8_t*)A, (float*)A, 512, 8192, P, A, A, W4_F16, 3584, 128, A, W4_BF16, nullptr, 0, nullptr), W4_OK, "w4a8 ws null");
  expect(w4a8_matmul_ws((int8_t*)A, (float*)A, 512, 8192, P, A, A, W4_F16, 3584, 128, A, W4_BF16, U, 4096, nullptr), W4_EINVAL, "w4a8 ws misaligned");
  expect(w4a8_matmul_ws((int8_t*)A, (float*)A, BIG, 8192, P, A, A, W4_F16, BIG, 128, A, W4_BF16, A, 4096, nullptr), W4_EINVAL, "w4a8 ws huge");
  expect(w4a8_matmul_ws((int8_t*)A, (float*)U, 1, 8192, P, A, A, W4_F16, 3584, 128, A, W4_BF16, A, 4096, nullptr), W4_OK, "w4a8 ws scale 4B");
  expect(w4a8_matmul_ws((int8_t*)A, (float*)(buf + 2), 1, 8192, P, A, A, W4_F16, 3584, 128, A, W4_BF16, A, 4096, nullptr), W4_EINVAL, "w4a8 ws scale 2B");
  expect((int)w4a8_matmul_workspace_size(BIG, BIG, BIG, 128), 0, "w4a8 ws size huge");
  expect((int)w4a8_matmul_workspace_size(512, 8192, 3584, 100), 0, "w4a8 ws size bad g");
  expect((int)w4a8_matmul_workspace_size(-1, 8192, 3584, 128), 0, "w4a8 ws size m<0");
  // GPTQ
  expect(gptq_hessian((const float*)A, 4096, 4096, (double*)A, nullptr), W4_OK, "hess ok");
  expect(gptq_hessian((const float*)A, BIG, 4096, (double*)A, nullptr), W4_EINVAL, "hess t huge");
  expect(gptq_hessian((const float*)A, 1, BIG, (double*)A, nullptr), W4_EINVAL, "hess k huge");
  expect(gptq_inverse_cholesky((double*)A, 4096, (double*)(buf + 16), (int32_t*)A, nullptr), W4_OK, "chol ok");
  expect(gptq_inverse_cholesky((double*)A, BIG, (double*)(buf + 16), (int32_t*)A, nullptr), W4_EINVAL, "chol huge");
  expect(gptq_quantize_pack_int4((float*)A, (const double*)A, 11008, 4096, 128, 0, P, A, A, W4_F16, nullptr), W4_OK, "sweep ok");
  expect(gptq_quantize_pack_int4((float*)A, (const double*)A, 4, 384, 96, 1, P, A, A, W4_F16, nullptr), W4_EINVAL, "sweep g96");
  expect(gptq_quantize_pack_int4((float*)A, (const double*)A, BIG, 4096, 128, 0, P, A, A, W4_F16, nullptr), W4_EINVAL, "sweep huge");
  // status strings
  for (int s = -5; s <= 2; ++s)
    if (w4_status_string(s) == nullptr) ++fails;
  std::printf("driver done, %d failure(s)\n", fails);
  return fails != 0;
}
'''


def test_abi_validation_under_sanitizers(tmp_path):
    (tmp_path / "stubs.cpp").write_text(_stubs())
    drv = tmp_path / "a" / "b"
    drv.mkdir(parents=True)
    (drv / "driver.cpp").write_text(DRIVER.replace("../../include/w4.h", os.path.join(ROOT, "include", "w4.h")))
    exe = tmp_path / "abi_san"
    flags = ["-std=c++17", "-g", "-O1", "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include", f"-I{CSRC}",
             "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
    cmd = ["g++", *flags, os.path.join(CSRC, "api.cpp"), str(tmp_path / "stubs.cpp"), str(drv / "driver.cpp"),
           f"-L{ROCM}/lib", "-lamdhip64", "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, LD_LIBRARY_PATH=f"{ROCM}/lib:" + os.environ.get("LD_LIBRARY_PATH", ""),
               ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0, (r.stdout + r.stderr)[-3000:]
    assert "driver done, 0 failure(s)" in r.stdout
