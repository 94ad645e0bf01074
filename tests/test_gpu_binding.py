"""The Python binding's argument checks: every tensor is checked for device, layout, type
and size before the library is called, and the library's own status codes come back
as NormError."""
import pytest

import row_normalization_norm_amd as rn

pytestmark = pytest.mark.gpu


def _tensors(device, M=8, N=256):
    import torch
    x = torch.randn(M, N, device=device).to(torch.bfloat16)
    return dict(x=x, g=torch.ones(N, dtype=torch.bfloat16, device=device),
                b=torch.zeros(N, dtype=torch.bfloat16, device=device), y=torch.empty_like(x),
                mean=torch.empty(M, device=device), rstd=torch.empty(M, device=device),
                dx=torch.empty_like(x), dg=torch.empty(N, device=device),
                db=torch.empty(N, device=device))


def test_forward_argument_checks(device):
    import torch
    t = _tensors(device)
    rn.norm_rms_fwd(t["x"], t["g"], t["y"], t["rstd"])  # valid
    with pytest.raises(ValueError, match="2-D"):
        rn.norm_rms_fwd(t["x"].view(-1), t["g"], t["y"], t["rstd"])
    with pytest.raises(ValueError, match="contiguous"):
        y = torch.empty(256, 8, dtype=torch.bfloat16, device=device).t()
        rn.norm_rms_fwd(t["x"], t["g"], y, t["rstd"])
    with pytest.raises(TypeError, match="must be"):
        rn.norm_rms_fwd(t["x"], t["g"], t["y"].float(), t["rstd"])
    with pytest.raises(ValueError, match="elements"):
        rn.norm_rms_fwd(t["x"], t["g"][:100], t["y"], t["rstd"])
    with pytest.raises(ValueError, match="elements"):
        rn.norm_ln_fwd(t["x"], t["g"], t["b"], t["y"], t["mean"][:3], t["rstd"])
    with pytest.raises(ValueError, match="cuda"):
        rn.norm_rms_fwd(t["x"], t["g"].cpu(), t["y"], t["rstd"])
    with pytest.raises(TypeError, match="float32"):
        rn.norm_rms_fwd(t["x"], t["g"].half(), t["y"], t["rstd"])
    # the library's own checks come back as NormError with its status
    with pytest.raises(rn.NormError) as e:
        rn.norm_rms_fwd(t["x"], t["g"], t["y"], t["rstd"], eps=-1.0)
    assert e.value.status == rn.NORM_ERR_BAD_EPS
    # fp32 gamma beside bf16 activations is a supported pair
    rn.norm_rms_fwd(t["x"], t["g"].float(), t["y"], t["rstd"])
    torch.cuda.synchronize(device)


def test_backward_argument_checks(device):
    import torch
    t = _tensors(device)
    rn.norm_ln_fwd(t["x"], t["g"], t["b"], t["y"], t["mean"], t["rstd"])
    rn.norm_ln_bwd(t["x"], t["x"], t["g"], t["mean"], t["rstd"], t["dx"], t["dg"], t["db"])
    with pytest.raises(TypeError, match="dgamma"):
        rn.norm_ln_bwd(t["x"], t["x"], t["g"], t["mean"], t["rstd"], t["dx"], t["dg"].half(),
                       t["db"])
    with pytest.raises(ValueError, match="dy"):
        rn.norm_rms_bwd(t["x"][:4], t["x"], t["g"], t["rstd"], t["dx"], t["dg"])
    with pytest.raises(ValueError, match="dx"):
        rn.norm_rms_bwd(t["x"], t["x"], t["g"], t["rstd"], t["dx"].t(), t["dg"])
    with pytest.raises(rn.NormError) as e:
        short = torch.empty(16, dtype=torch.uint8, device=device)
        rn.norm_ln_bwd(t["x"], t["x"], t["g"], t["mean"], t["rstd"], t["dx"], t["dg"], t["db"],
                       workspace=short)
    assert e.value.status == rn.NORM_ERR_WORKSPACE_TOO_SMALL
    torch.cuda.synchronize(device)
