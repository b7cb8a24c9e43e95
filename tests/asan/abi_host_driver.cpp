// Host-side driver of the C ABI in include/moe.h for the AddressSanitizer build of api.cpp.
//
// Every call below returns from api.cpp's validation (shape, dtype, pointers, ring head,
// workspace size, static scratch limit) before any HIP call, so the driver needs no GPU.
// The pointers handed in are host addresses that api.cpp must never dereference; the
// shape struct is the only memory it reads.  Exit status 0 when every call returned the
// status the header documents; the sanitizer ends the process with its own report on
// any invalid access.
#include <cstdio>
#include <cstring>

#include "moe.h"

namespace {

int failures = 0;

void expect(const char* what, long got, long want) {
  if (got != want) {
    std::printf("FAIL %s: got %ld, want %ld\n", what, got, want);
    ++failures;
  }
}

unsigned char fake_buf[64];
void* const P = fake_buf;
int32_t* const PI = reinterpret_cast<int32_t*>(fake_buf);
float* const PF = reinterpret_cast<float*>(fake_buf);
uint8_t* const PB = fake_buf;

// A shape on the heap, exactly sizeof(moe_shape) bytes: a read past its end is reported.
moe_shape* heap_shape(int64_t T, int d, int E, int k, int f, int dtype, int64_t C = -1,
                      int fs = 0) {
  moe_shape* s = new moe_shape;
  s->tokens = T;
  s->capacity = C < 0 ? T * k : C;
  s->hidden = d;
  s->experts = E;
  s->top_k = k;
  s->ffn = f;
  s->shared_ffn = fs;
  s->dtype = dtype;
  return s;
}

void shape_checks() {
  expect("check_shape(NULL)", moe_check_shape(nullptr), MOE_ERR_NULL);
  struct Case {
    const char* name;
    int64_t T;
    int d, E, k, f, dtype;
    int64_t C;
    int want;
  } cases[] = {
      {"bf16 ok", 2048, 7168, 256, 8, 2048, MOE_BF16, -1, MOE_OK},
      {"mx ok", 2048, 7168, 256, 8, 2048, MOE_MXFP8, -1, MOE_OK},
      {"f32 ok", 100, 72, 16, 4, 40, MOE_F32, -1, MOE_OK},
      {"no tokens", 0, 256, 8, 2, 128, MOE_BF16, 0, MOE_OK},
      {"bad dtype", 16, 256, 8, 2, 128, 7, -1, MOE_ERR_DTYPE},
      {"negative T", -1, 256, 8, 2, 128, MOE_BF16, 0, MOE_ERR_SHAPE},
      {"d 0", 16, 0, 8, 2, 128, MOE_BF16, -1, MOE_ERR_SHAPE},
      {"k > E", 16, 256, 4, 5, 128, MOE_BF16, -1, MOE_ERR_SHAPE},
      {"k 0", 16, 256, 4, 0, 128, MOE_BF16, 16, MOE_ERR_SHAPE},
      {"k > 32", 16, 256, 64, 33, 128, MOE_BF16, -1, MOE_ERR_SHAPE},
      {"E > 1024", 16, 256, 1025, 2, 128, MOE_BF16, -1, MOE_ERR_SHAPE},
      {"T > 2^30", (int64_t)1 << 31, 256, 8, 1, 128, MOE_BF16, -1, MOE_ERR_SHAPE},
      {"bf16 d % 64", 16, 96, 8, 2, 128, MOE_BF16, -1, MOE_ERR_SHAPE},
      {"mx f % 128", 16, 256, 8, 2, 192, MOE_MXFP8, -1, MOE_ERR_SHAPE},
      {"capacity short", 16, 256, 8, 2, 128, MOE_BF16, 31, MOE_ERR_CAPACITY},
      {"capacity > 2^31-1", 16, 256, 8, 2, 128, MOE_BF16, (int64_t)1 << 31, MOE_ERR_SHAPE},
      // rows of d * 2 = 14,336 bytes: the first capacity whose ring reaches 4 GiB, and the last below
      {"ring of 4 GiB", 16, 7168, 8, 2, 128, MOE_BF16, (((int64_t)1 << 32) + 14335) / 14336,
       MOE_ERR_SHAPE},
      {"ring below 4 GiB", 16, 7168, 8, 2, 128, MOE_BF16, (((int64_t)1 << 32) + 14335) / 14336 - 1,
       MOE_OK},
  };
  for (const Case& c : cases) {
    moe_shape* s = heap_shape(c.T, c.d, c.E, c.k, c.f, c.dtype, c.C);
    expect(c.name, moe_check_shape(s), c.want);
    for (int op = 0; op <= MOE_OP_FORWARD + 1; ++op) {
      const size_t ws = moe_workspace_bytes(s, op);
      if (c.want != MOE_OK) expect("workspace of an invalid shape", (long)ws, 0);
      if (ws % 256) expect("workspace multiple of 256", (long)(ws % 256), 0);
    }
    delete s;
  }
  expect("workspace(NULL)", (long)moe_workspace_bytes(nullptr, MOE_OP_ROUTE), 0);
  moe_shape* s = heap_shape(2048, 7168, 256, 8, 2048, MOE_BF16);
  expect("workspace unknown op", (long)moe_workspace_bytes(s, 99), 0);
  expect("workspace forward bf16 > 0", moe_workspace_bytes(s, MOE_OP_FORWARD) > 0, 1);
  expect("workspace backward > 0", moe_workspace_bytes(s, MOE_OP_BACKWARD) > 0, 1);
  s->dtype = MOE_MXFP8;
  expect("workspace forward mx", (long)moe_workspace_bytes(s, MOE_OP_FORWARD), 0);
  expect("workspace backward mx > 0", moe_workspace_bytes(s, MOE_OP_BACKWARD) > 0, 1);
  delete s;
}

void status_strings() {
  for (int st = -2; st <= MOE_ERR_SCRATCH + 2; ++st) {
    const char* m = moe_status_string(st);
    expect("status string non-null", m != nullptr, 1);
    if (m) expect("status string non-empty", std::strlen(m) > 0, 1);
  }
}

void route_dispatch_ffn_combine() {
  moe_shape* s = heap_shape(64, 256, 8, 2, 128, MOE_BF16);
  const size_t wr = moe_workspace_bytes(s, MOE_OP_ROUTE);
  expect("route NULL x", moe_route(s, nullptr, PF, nullptr, PI, PF, PI, P, wr, nullptr),
         MOE_ERR_NULL);
  expect("route NULL w_router", moe_route(s, P, nullptr, nullptr, PI, PF, PI, P, wr, nullptr),
         MOE_ERR_NULL);
  expect("route small workspace", moe_route(s, P, PF, nullptr, PI, PF, PI, P, wr - 1, nullptr),
         MOE_ERR_WORKSPACE);
  const size_t wd = moe_workspace_bytes(s, MOE_OP_DISPATCH);
  expect("dispatch head = C",
         moe_dispatch(s, P, PI, s->capacity, P, nullptr, PI, PI, PI, P, wd, nullptr),
         MOE_ERR_SHAPE);
  expect("dispatch head < 0", moe_dispatch(s, P, PI, -1, P, nullptr, PI, PI, PI, P, wd, nullptr),
         MOE_ERR_SHAPE);
  expect("dispatch NULL slot_copy",
         moe_dispatch(s, P, PI, 0, P, nullptr, PI, PI, nullptr, P, wd, nullptr), MOE_ERR_NULL);
  expect("dispatch small workspace",
         moe_dispatch(s, P, PI, 0, P, nullptr, PI, PI, PI, P, wd - 1, nullptr),
         MOE_ERR_WORKSPACE);
  const size_t wf = moe_workspace_bytes(s, MOE_OP_EXPERT_FFN);
  expect("ffn NULL w_down",
         moe_expert_ffn(s, P, nullptr, PI, 0, P, P, nullptr, nullptr, nullptr, nullptr, P,
                        nullptr, P, wf, nullptr),
         MOE_ERR_NULL);
  expect("ffn small workspace",
         moe_expert_ffn(s, P, nullptr, PI, 0, P, P, P, nullptr, nullptr, nullptr, P, nullptr, P,
                        wf - 1, nullptr),
         MOE_ERR_WORKSPACE);
  expect("combine NULL y", moe_combine(s, P, PI, PF, nullptr, nullptr), MOE_ERR_NULL);
  s->dtype = MOE_MXFP8;
  const size_t wdm = moe_workspace_bytes(s, MOE_OP_DISPATCH);
  expect("dispatch mx NULL scale",
         moe_dispatch(s, P, PI, 0, P, nullptr, PI, PI, PI, P, wdm, nullptr), MOE_ERR_NULL);
  const size_t wfm = moe_workspace_bytes(s, MOE_OP_EXPERT_FFN);
  expect("ffn mx NULL weight scale",
         moe_expert_ffn(s, P, PB, PI, 0, P, P, P, PB, nullptr, PB, P, nullptr, P, wfm, nullptr),
         MOE_ERR_NULL);
  s->dtype = MOE_F32;
  const size_t wff = moe_workspace_bytes(s, MOE_OP_EXPERT_FFN);
  expect("ffn f32 saved A|U",
         moe_expert_ffn(s, P, nullptr, PI, 0, P, P, P, nullptr, nullptr, nullptr, P, P, P, wff,
                        nullptr),
         MOE_ERR_DTYPE);
  delete s;
}

void forward_decode() {
  moe_shape* s = heap_shape(64, 256, 8, 2, 128, MOE_BF16);
  const size_t wf = moe_workspace_bytes(s, MOE_OP_FORWARD);
  expect("forward NULL ring_y",
         moe_forward(s, P, PF, nullptr, P, P, P, 0, PI, PF, PI, P, PI, PI, PI, nullptr, nullptr,
                     P, 0, P, wf, nullptr),
         MOE_ERR_NULL);
  expect("forward head = C",
         moe_forward(s, P, PF, nullptr, P, P, P, s->capacity, PI, PF, PI, P, PI, PI, PI, P,
                     nullptr, P, 0, P, wf, nullptr),
         MOE_ERR_SHAPE);
  expect("forward small workspace",
         moe_forward(s, P, PF, nullptr, P, P, P, 0, PI, PF, PI, P, PI, PI, PI, P, nullptr, P, 0,
                     P, wf - 1, nullptr),
         MOE_ERR_WORKSPACE);
  s->dtype = MOE_MXFP8;
  expect("forward mx", moe_forward(s, P, PF, nullptr, P, P, P, 0, PI, PF, PI, P, PI, PI, PI, P,
                                   nullptr, P, 0, P, 1 << 30, nullptr),
         MOE_ERR_DTYPE);
  delete s;

  moe_shape* d = heap_shape(8, 7168, 256, 8, 2048, MOE_BF16, -1, 2048);
  const size_t wdec = moe_workspace_bytes(d, MOE_OP_DECODE);
  expect("decode small workspace",
         moe_decode(d, P, PF, nullptr, P, P, P, P, P, P, P, PI, PF, P, wdec - 1, nullptr),
         MOE_ERR_WORKSPACE);
  expect("decode NULL shared weight",
         moe_decode(d, P, PF, nullptr, P, P, P, nullptr, P, P, P, PI, PF, P, wdec, nullptr),
         MOE_ERR_NULL);
  expect("decode_noalloc NULL y",
         moe_decode_noalloc(d, P, PF, nullptr, P, P, P, P, P, P, nullptr, PI, PF, nullptr),
         MOE_ERR_NULL);
  d->tokens = 9;
  d->capacity = 72;
  expect("decode B 9", moe_decode(d, P, PF, nullptr, P, P, P, P, P, P, P, PI, PF, P, wdec, nullptr),
         MOE_ERR_SHAPE);
  delete d;
  moe_shape* big = heap_shape(8, 1024, 64, 16, 4096, MOE_BF16, -1, 4096);
  expect("decode_noalloc beyond scratch",
         moe_decode_noalloc(big, P, PF, nullptr, P, P, P, P, P, P, P, PI, PF, nullptr),
         MOE_ERR_SCRATCH);
  big->shared_ffn = 1024;
  expect("decode shared width != f",
         moe_decode_noalloc(big, P, PF, nullptr, P, P, P, P, P, P, P, PI, PF, nullptr),
         MOE_ERR_SHAPE);
  delete big;
}

void backward() {
  moe_shape* s = heap_shape(64, 256, 8, 2, 128, MOE_BF16);
  const size_t wb = moe_workspace_bytes(s, MOE_OP_BACKWARD);
  expect("backward NULL saved_au",
         moe_backward(s, P, P, PF, PI, PF, P, PI, PI, PI, 0, nullptr, P, P, P, P, P, P, P, PF, P,
                      wb, nullptr),
         MOE_ERR_NULL);
  expect("backward small workspace",
         moe_backward(s, P, P, PF, PI, PF, P, PI, PI, PI, 0, P, P, P, P, P, P, P, P, PF, P,
                      wb - 1, nullptr),
         MOE_ERR_WORKSPACE);
  expect("backward_mx on bf16",
         moe_backward_mx(s, P, P, PF, PI, PF, PI, PI, PI, 0, P, PB, PB, PB, PB, P, P, P, P, PF, P,
                         wb, nullptr),
         MOE_ERR_DTYPE);
  s->hidden = 192;   // a multiple of 64 but not of 128
  expect("backward d % 128",
         moe_backward(s, P, P, PF, PI, PF, P, PI, PI, PI, 0, P, P, P, P, P, P, P, P, PF, P,
                      1 << 30, nullptr),
         MOE_ERR_SHAPE);
  s->hidden = 256;
  s->dtype = MOE_MXFP8;
  const size_t wbm = moe_workspace_bytes(s, MOE_OP_BACKWARD);
  expect("backward on mx",
         moe_backward(s, P, P, PF, PI, PF, P, PI, PI, PI, 0, P, P, P, P, P, P, P, P, PF, P, wbm,
                      nullptr),
         MOE_ERR_DTYPE);
  expect("backward_mx NULL transposed scale",
         moe_backward_mx(s, P, P, PF, PI, PF, PI, PI, PI, 0, P, PB, nullptr, PB, PB, P, P, P, P,
                         PF, P, wbm, nullptr),
         MOE_ERR_NULL);
  expect("backward_mx head = C",
         moe_backward_mx(s, P, P, PF, PI, PF, PI, PI, PI, s->capacity, P, PB, PB, PB, PB, P, P, P,
                         P, PF, P, wbm, nullptr),
         MOE_ERR_SHAPE);
  expect("backward_mx small workspace",
         moe_backward_mx(s, P, P, PF, PI, PF, PI, PI, PI, 0, P, PB, PB, PB, PB, P, P, P, P, PF, P,
                         wbm - 1, nullptr),
         MOE_ERR_WORKSPACE);
  delete s;
}

void quantizers() {
  expect("quantize_mx NULL", moe_quantize_mx(nullptr, 4, 128, PB, PB, nullptr), MOE_ERR_NULL);
  expect("quantize_mx cols % 128", moe_quantize_mx(P, 4, 96, PB, PB, nullptr), MOE_ERR_SHAPE);
  expect("quantize_mx rows < 0", moe_quantize_mx(P, -1, 128, PB, PB, nullptr), MOE_ERR_SHAPE);
  expect("quantize_mx_t rows % 32", moe_quantize_mx_t(P, 1, 48, 128, PB, 128, 0, PB, nullptr),
         MOE_ERR_SHAPE);
  expect("quantize_mx_t ld % 128", moe_quantize_mx_t(P, 1, 64, 128, PB, 96, 0, PB, nullptr),
         MOE_ERR_SHAPE);
  expect("quantize_mx_t col0 + rows > ld",
         moe_quantize_mx_t(P, 1, 64, 128, PB, 128, 96, PB, nullptr), MOE_ERR_SHAPE);
  expect("quantize_mx_t NULL scales", moe_quantize_mx_t(P, 1, 64, 128, PB, 128, 0, nullptr,
                                                        nullptr),
         MOE_ERR_NULL);
  expect("quantize_mx_both NULL transposed scales",
         moe_quantize_mx_both(P, 1, 128, 128, PB, PB, PB, 128, 0, nullptr, nullptr), MOE_ERR_NULL);
  expect("quantize_mx_both rows % 128",
         moe_quantize_mx_both(P, 1, 96, 128, PB, PB, PB, 128, 0, PB, nullptr), MOE_ERR_SHAPE);
  expect("quantize_mx_both col0 % 128",
         moe_quantize_mx_both(P, 1, 128, 128, PB, PB, PB, 256, 64, PB, nullptr), MOE_ERR_SHAPE);
  expect("quantize_mx_both col0 + rows > ld",
         moe_quantize_mx_both(P, 1, 256, 128, PB, PB, PB, 128, 0, PB, nullptr), MOE_ERR_SHAPE);
}

}  // namespace

int main() {
  shape_checks();
  status_strings();
  route_dispatch_ffn_combine();
  forward_decode();
  backward();
  quantizers();
  std::printf("%s: %d failure(s)\n", failures ? "FAILED" : "ok", failures);
  return failures ? 1 : 0;
}
